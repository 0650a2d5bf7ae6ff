"""Torch-facing wrappers with the C ABI's names (bsa_estimate_mask, bsa_forward, ...).

Argument marshalling only: shapes, dtypes and devices are checked, outputs and
workspaces are allocated as torch tensors when the caller does not pass them,
and the call goes to libbsa.so on torch's current HIP stream.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import (BSA_BF16, BSA_FP32, BSA_WS_BACKWARD, BSA_WS_ESTIMATE, BSA_WS_ESTIMATE_HIER, BSA_WS_FORWARD,
                   BSA_WS_SELECT_FROM_MASS,
                   BSA_WS_STRUCTURED, BsaCsr, BsaPatternParams, BsaShape,
                   check, load)


@dataclass
class Csr:
    """Block mask: row_ptr [R+1] and col_idx [capacity], int32 device tensors."""
    row_ptr: torch.Tensor
    col_idx: torch.Tensor

    @property
    def capacity(self) -> int:
        return self.col_idx.numel()

    def c(self) -> BsaCsr:
        return BsaCsr(self.row_ptr.data_ptr(), self.col_idx.data_ptr() if self.capacity else None, self.capacity)

    def nnz(self) -> int:
        """Total selected blocks (reads row_ptr[R]; synchronises)."""
        return int(self.row_ptr[-1].item())

    def to_host(self):
        """(row_ptr, col_idx[:nnz]) as int64 numpy arrays."""
        rp = self.row_ptr.cpu().numpy().astype("int64")
        n = min(int(rp[-1]), self.capacity)
        return rp, self.col_idx[:n].cpu().numpy().astype("int64")


def csr_from_host(row_ptr, col_idx, device, capacity: int | None = None) -> Csr:
    rp = torch.as_tensor(row_ptr, dtype=torch.int32).to(device)
    ci = torch.as_tensor(col_idx, dtype=torch.int32)
    cap = ci.numel() if capacity is None else capacity
    buf = torch.zeros(max(cap, 1), dtype=torch.int32)
    buf[: min(cap, ci.numel())] = ci[:cap]
    return Csr(rp, buf[:cap].to(device) if cap else buf[:0].to(device))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BSA_BF16
    if t.dtype == torch.float32:
        return BSA_FP32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def make_shape(B: int, H: int, N: int, D: int, block: int, dtype: int) -> BsaShape:
    return BsaShape(B, H, N, D, block, dtype)


def _shape_of(q: torch.Tensor, block: int) -> BsaShape:
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, D]")
    B, H, N, D = q.shape
    return make_shape(B, H, N, D, block, _dtype_code(q))


def _check(t: torch.Tensor, name: str, like: torch.Tensor | None = None, dtype=None, shape=None, device=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if like is not None and (t.shape != like.shape or t.dtype != like.dtype or t.device != like.device):
        raise ValueError(f"{name} must match q in shape, dtype and device")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on q's device")


def _check_csr(m: Csr, rows: int, name: str, device) -> None:
    """The library reads row_ptr[0..rows] and at most capacity col_idx entries."""
    for t, part in ((m.row_ptr, "row_ptr"), (m.col_idx, "col_idx")):
        if t.dtype != torch.int32 or t.device != device or not t.is_contiguous():
            raise ValueError(f"{name}.{part} must be a contiguous int32 tensor on q's device")
    if m.row_ptr.numel() < rows + 1:
        raise ValueError(f"{name}.row_ptr must hold B*H*nb + 1 = {rows + 1} entries")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def bsa_workspace_size(shape: BsaShape, kind: int, capacity: int = 0) -> int:
    return int(load().bsa_workspace_size(ctypes.byref(shape), kind, capacity))


def _workspace(shape: BsaShape, kind: int, capacity: int, ws: torch.Tensor | None, device) -> torch.Tensor:
    """The caller's workspace, or a new one of the size the library asks for.
    The library itself checks that it is large enough (sizes in bytes)."""
    if ws is None:
        need = bsa_workspace_size(shape, kind, capacity)
        return torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    if ws.device != device or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's device")
    return ws


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def num_rows(q: torch.Tensor, block: int) -> int:
    B, H, N, _ = q.shape
    return B * H * (-(-N // block))


def bsa_estimate_mask(q: torch.Tensor, k: torch.Tensor, top_p: float, block: int, scale: float = 0.0,
                      candidate: Csr | None = None, keep_prefix_tokens: int = 0, out: Csr | None = None,
                      capacity: int | None = None, workspace: torch.Tensor | None = None,
                      sub_blocks: int = 1) -> Csr:
    """Block-importance estimator -> CSR mask (see bsa_estimate_mask in include/bsa.h).
    ``sub_blocks`` > 1 selects hierarchical block scoring
    (bsa_estimate_mask_hierarchical): block logits as the log-sum-exp over
    that many key sub-blocks."""
    _check(q, "q")
    _check(k, "k", like=q)
    shape = _shape_of(q, block)
    nb = -(-q.shape[2] // block)
    R = num_rows(q, block)
    if out is None:
        cap = R * nb if capacity is None else capacity
        out = Csr(torch.empty(R + 1, dtype=torch.int32, device=q.device),
                  torch.empty(cap, dtype=torch.int32, device=q.device))
    _check_csr(out, R, "out", q.device)
    if candidate is not None:
        _check_csr(candidate, R, "candidate", q.device)
    cand = ctypes.byref(candidate.c()) if candidate is not None else None
    oc = out.c()
    if sub_blocks == 1:
        ws = _workspace(shape, BSA_WS_ESTIMATE, 0, workspace, q.device)
        st = load().bsa_estimate_mask(ctypes.byref(shape), q.data_ptr(), k.data_ptr(), float(top_p), float(scale),
                                      cand, int(keep_prefix_tokens), ctypes.byref(oc), ws.data_ptr(), _nbytes(ws),
                                      _stream())
        check(st, "bsa_estimate_mask")
    else:
        ws = _workspace(shape, BSA_WS_ESTIMATE_HIER, 0, workspace, q.device)
        st = load().bsa_estimate_mask_hierarchical(ctypes.byref(shape), q.data_ptr(), k.data_ptr(), float(top_p),
                                                   float(scale), cand, int(keep_prefix_tokens), int(sub_blocks),
                                                   ctypes.byref(oc), ws.data_ptr(), _nbytes(ws), _stream())
        check(st, "bsa_estimate_mask_hierarchical")
    return out


def bsa_select_from_mass(q: torch.Tensor, mask: Csr, mass: torch.Tensor, top_p: float, block: int,
                         keep_prefix_tokens: int = 0, out: Csr | None = None,
                         workspace: torch.Tensor | None = None) -> Csr:
    """Mask narrowing: Top-p over the block masses aligned with ``mask`` -> CSR
    (see bsa_select_from_mass in include/bsa.h).  ``q`` supplies the shape only."""
    _check(q, "q")
    _check(mass, "mass", dtype=torch.float32, device=q.device)
    if mass.numel() < mask.capacity:
        raise ValueError("mass must hold mask.capacity entries")
    shape = _shape_of(q, block)
    nb = -(-q.shape[2] // block)
    R = num_rows(q, block)
    if out is None:
        out = Csr(torch.empty(R + 1, dtype=torch.int32, device=q.device),
                  torch.empty(R * nb, dtype=torch.int32, device=q.device))
    _check_csr(mask, R, "mask", q.device)
    _check_csr(out, R, "out", q.device)
    ws = _workspace(shape, BSA_WS_SELECT_FROM_MASS, 0, workspace, q.device)
    mc, oc = mask.c(), out.c()
    st = load().bsa_select_from_mass(ctypes.byref(shape), ctypes.byref(mc), mass.data_ptr(), float(top_p),
                                     int(keep_prefix_tokens), ctypes.byref(oc), ws.data_ptr(), _nbytes(ws),
                                     _stream())
    check(st, "bsa_select_from_mass")
    return out


def bsa_select_from_mass_noalloc(q: torch.Tensor, mask: Csr, mass: torch.Tensor, top_p: float, block: int,
                                 keep_prefix_tokens: int = 0, out: Csr | None = None) -> Csr:
    """Mask narrowing without a workspace (bsa_select_from_mass_noalloc in
    include/bsa.h): the library's per-GPU static scratch replaces the
    workspace; ``out`` should be preallocated by callers that cannot allocate."""
    _check(q, "q")
    _check(mass, "mass", dtype=torch.float32, device=q.device)
    if mass.numel() < mask.capacity:
        raise ValueError("mass must hold mask.capacity entries")
    shape = _shape_of(q, block)
    nb = -(-q.shape[2] // block)
    R = num_rows(q, block)
    if out is None:
        out = Csr(torch.empty(R + 1, dtype=torch.int32, device=q.device),
                  torch.empty(R * nb, dtype=torch.int32, device=q.device))
    _check_csr(mask, R, "mask", q.device)
    _check_csr(out, R, "out", q.device)
    mc, oc = mask.c(), out.c()
    st = load().bsa_select_from_mass_noalloc(ctypes.byref(shape), ctypes.byref(mc), mass.data_ptr(), float(top_p),
                                             int(keep_prefix_tokens), ctypes.byref(oc), _stream())
    check(st, "bsa_select_from_mass_noalloc")
    return out


def bsa_structured_mask(q: torch.Tensor, head_kind: torch.Tensor, block: int, prefix_tokens: int = 0,
                        frame_tokens: int = 1, band: int = 0, period: int = 1, stripes: torch.Tensor | None = None,
                        out: Csr | None = None, workspace: torch.Tensor | None = None) -> Csr:
    """Structured head masks -> CSR (see bsa_structured_mask in include/bsa.h).
    ``q`` supplies the shape only; ``head_kind`` is an int32 device tensor of B*H pattern codes."""
    _check(q, "q")
    B, H, N, _ = q.shape
    if head_kind.dtype != torch.int32 or head_kind.numel() != B * H or head_kind.device != q.device:
        raise ValueError("head_kind must be an int32 tensor of B*H entries on q's device")
    head_kind = head_kind.contiguous()
    if stripes is not None:
        if stripes.dtype != torch.int32 or stripes.device != q.device:
            raise ValueError("stripes must be an int32 tensor on q's device")
        stripes = stripes.contiguous()
    shape = _shape_of(q, block)
    nb = -(-N // block)
    R = num_rows(q, block)
    if out is None:
        out = Csr(torch.empty(R + 1, dtype=torch.int32, device=q.device),
                  torch.empty(R * nb, dtype=torch.int32, device=q.device))
    _check_csr(out, R, "out", q.device)
    ws = _workspace(shape, BSA_WS_STRUCTURED, 0, workspace, q.device)
    prm = BsaPatternParams(int(prefix_tokens), int(frame_tokens), int(band), int(period),
                           stripes.data_ptr() if stripes is not None and stripes.numel() else None,
                           int(stripes.numel()) if stripes is not None else 0)
    oc = out.c()
    st = load().bsa_structured_mask(ctypes.byref(shape), head_kind.data_ptr(), ctypes.byref(prm), ctypes.byref(oc),
                                    ws.data_ptr(), _nbytes(ws), _stream())
    check(st, "bsa_structured_mask")
    return out


def bsa_permute_tokens(x: torch.Tensor, perm: torch.Tensor, inverse: bool = False,
                       out: torch.Tensor | None = None) -> torch.Tensor:
    """Token permutation of a [B, H, N, ...] tensor along N (see bsa_permute_rows
    in include/bsa.h): gather out[:, :, t] = x[:, :, perm[t]], or with
    ``inverse`` the scatter out[:, :, perm[t]] = x[:, :, t]."""
    if not x.is_contiguous() or x.dim() < 3:
        raise ValueError("x must be a contiguous [B, H, N, ...] tensor")
    n = x.shape[2]
    if perm.dtype != torch.int32 or perm.numel() != n or perm.device != x.device:
        raise ValueError("perm must be an int32 tensor of N entries on x's device")
    perm = perm.contiguous()
    out = torch.empty_like(x) if out is None else out
    if out.shape != x.shape or out.dtype != x.dtype or out.device != x.device or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like x on x's device")
    heads = x.shape[0] * x.shape[1]
    row_bytes = x.element_size() * (x.numel() // max(1, heads * n))
    st = load().bsa_permute_rows(int(heads), int(n), int(row_bytes), x.data_ptr(), perm.data_ptr(), int(bool(inverse)),
                                 out.data_ptr(), _stream())
    check(st, "bsa_permute_rows")
    return out


def bsa_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mask: Csr, block: int, scale: float = 0.0,
                want_mass: bool = True, out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                mass: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                o32: torch.Tensor | None = None):
    """Sparse attention forward -> (O, LSE, block mass or None).  ``o32``: an
    optional [B, H, N, D] fp32 tensor that receives O before its rounding to
    bf16 (bf16 data only), for the single-pass delta of bsa_backward."""
    _check(q, "q")
    _check(k, "k", like=q)
    _check(v, "v", like=q)
    shape = _shape_of(q, block)
    B, H, N, D = q.shape
    o = torch.empty_like(q) if out is None else out
    _check(o, "out", like=q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check(lse, "lse", dtype=torch.float32, shape=(B, H, N), device=q.device)
    _check_csr(mask, num_rows(q, block), "mask", q.device)
    if want_mass and mass is None:
        mass = torch.empty(max(mask.capacity, 1), dtype=torch.float32, device=q.device)
    if mass is not None:
        _check(mass, "mass", dtype=torch.float32, device=q.device)
        if mass.numel() < mask.capacity:
            raise ValueError("mass must hold mask.capacity entries")
    if o32 is not None:
        _check(o32, "o32", dtype=torch.float32, shape=q.shape, device=q.device)
    ws = _workspace(shape, BSA_WS_FORWARD, mask.capacity, workspace, q.device)
    mc = mask.c()
    st = load().bsa_forward(ctypes.byref(shape), q.data_ptr(), k.data_ptr(), v.data_ptr(), float(scale),
                            ctypes.byref(mc), o.data_ptr(), lse.data_ptr(), _ptr(mass), _ptr(o32), ws.data_ptr(),
                            _nbytes(ws), _stream())
    check(st, "bsa_forward")
    return o, lse, (mass[: mask.capacity] if mass is not None else None)


def bsa_backward(q, k, v, o, d_o, lse, mask: Csr, block: int, scale: float = 0.0,
                 workspace: torch.Tensor | None = None, dq=None, dk=None, dv=None, o32=None):
    """Backward of bsa_forward for dL/dO = d_o -> (dQ, dK, dV).  ``o32``: the
    forward's fp32 O (bf16 data only) -> delta from it and a single dQ pass."""
    _check(q, "q")
    for t, n in ((k, "k"), (v, "v"), (o, "o"), (d_o, "d_o")):
        _check(t, n, like=q)
    shape = _shape_of(q, block)
    _check(lse, "lse", dtype=torch.float32, shape=q.shape[:3], device=q.device)
    _check_csr(mask, num_rows(q, block), "mask", q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check(t, n, like=q)
    if o32 is not None:
        _check(o32, "o32", dtype=torch.float32, shape=q.shape, device=q.device)
    ws = _workspace(shape, BSA_WS_BACKWARD, mask.capacity, workspace, q.device)
    mc = mask.c()
    st = load().bsa_backward(ctypes.byref(shape), q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                             _ptr(o32), d_o.data_ptr(), lse.data_ptr(), float(scale), ctypes.byref(mc), dq.data_ptr(),
                             dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), _nbytes(ws), _stream())
    check(st, "bsa_backward")
    return dq, dk, dv


def bsa_status_string(status: int) -> str:
    return load().bsa_status_string(status).decode()


def bsa_last_error() -> str:
    return load().bsa_last_error().decode()


def bsa_version() -> int:
    return int(load().bsa_version())
