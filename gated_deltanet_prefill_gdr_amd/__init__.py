"""Chunked gated delta rule prefill for AMD MI355X (gfx950): thin Python binding.

The computation runs entirely in the HIP kernels of ``libgdr.so`` behind the C ABI declared in
``include/gdr.h``. This module only marshals arguments: it checks torch tensors (device,
dtype, shape, contiguity), allocates the outputs and the workspace with torch, converts a 0/1
right-pad mask into per-row lengths, and passes raw device pointers plus torch's current HIP
stream down. There is no fallback: if the library is missing, every call raises.

    o, s_final = prefill(q, k, v, g, beta, valid=None, s0=None, s0_row=None)

q, k [B, L, Hk, 128]; v [B, L, Hv, 128] (float32 or bfloat16, same dtype); g [B, L, Hv]
float32; beta [B, L, Hv] float32 or q's dtype; valid: None, int32 lengths [B], or a 0/1 mask
[B, L] that is 1 then 0 along each row; s0 [n_s0, Hv, 128, 128] float32; s0_row [B] int32.
Returns o [B, L, Hv, 128] in v's dtype and s_final [B, Hv, 128, 128] float32 (None if
``want_state`` is False).
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["prefill", "workspace_size", "check", "last_error", "library", "timing_enable",
           "timing_read", "kernel_name", "GdrError", "KERNELS", "LIB_PATH", "decode"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdr.so")
HEAD_DIM = 128
GDR_F32, GDR_BF16 = 0, 1
STATUS = {0: "GDR_OK", -1: "GDR_EINVAL", -2: "GDR_EUNSUPPORTED", -3: "GDR_EWORKSPACE", -4: "GDR_EHIP"}
KERNELS = ("gdr_prep", "gdr_scan", "gdr_transition", "gdr_combine", "gdr_decode")


class GdrError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class Desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "L", "Hk", "Hv", "Dk", "Dv", "n_s0", "qkv_dtype", "beta_dtype")]


_lib = None


def library() -> ctypes.CDLL:
    """Load libgdr.so (built by build.py); raises if it is not there."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with gated_deltanet_prefill_gdr_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.gdr_prefill_workspace_size.argtypes = [ctypes.POINTER(Desc)]
    lib.gdr_prefill_workspace_size.restype = sz
    lib.gdr_prefill_check.argtypes = [ctypes.POINTER(Desc)] + [vp] * 11 + [sz]
    lib.gdr_prefill_check.restype = i32
    lib.gdr_prefill.argtypes = [ctypes.POINTER(Desc)] + [vp] * 11 + [sz, vp]
    lib.gdr_prefill.restype = i32
    lib.gdr_decode.argtypes = [ctypes.POINTER(Desc)] + [vp] * 10 + [vp]
    lib.gdr_decode.restype = i32
    lib.gdr_last_error.argtypes = []
    lib.gdr_last_error.restype = ctypes.c_char_p
    lib.gdr_timing_enable.argtypes = [i32]
    lib.gdr_timing_enable.restype = i32
    lib.gdr_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64), i32]
    lib.gdr_timing_read.restype = i32
    lib.gdr_kernel_name.argtypes = [i32]
    lib.gdr_kernel_name.restype = ctypes.c_char_p
    _lib = lib
    return lib


def last_error() -> str:
    return library().gdr_last_error().decode()


def _raise(status: int):
    if status != 0:
        raise GdrError(status, last_error())


def make_desc(B, L, Hk, Hv, n_s0=0, qkv_bf16=False, beta_bf16=False, Dk=HEAD_DIM, Dv=HEAD_DIM) -> Desc:
    return Desc(B, L, Hk, Hv, Dk, Dv, n_s0, GDR_BF16 if qkv_bf16 else GDR_F32,
                GDR_BF16 if beta_bf16 else GDR_F32)


def workspace_size(desc: Desc) -> int:
    n = library().gdr_prefill_workspace_size(ctypes.byref(desc))
    if n == ctypes.c_size_t(-1).value:
        raise GdrError(-1, last_error())
    return n


def check(desc: Desc, ptrs, ws_bytes: int) -> int:
    """Host-only validation (status code); ptrs = 11 integers in C-ABI order (0 = NULL)."""
    return library().gdr_prefill_check(ctypes.byref(desc), *[p or None for p in ptrs], ws_bytes)


def kernel_name(i: int) -> str:
    return library().gdr_kernel_name(i).decode()


def timing_enable(on: bool = True):
    _raise(library().gdr_timing_enable(1 if on else 0))


def timing_read():
    """{kernel name: (total ms, launches)} since the last read (waits for the events)."""
    n = len(KERNELS)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    _raise(library().gdr_timing_read(ms, cnt, n))
    return {KERNELS[i]: (ms[i], cnt[i]) for i in range(n)}


def _ptr(t):
    return 0 if t is None else t.data_ptr()


def _lengths_from_valid(valid, B, L, device):
    import torch
    if valid is None:
        return None
    if valid.dtype == torch.int32 and valid.dim() == 1:
        if valid.shape[0] != B:
            raise ValueError(f"lengths must have shape [{B}]")
        if valid.device.type == "cpu":
            if valid.numel() and (int(valid.min()) < 0 or int(valid.max()) > L):
                raise ValueError(f"lengths must lie in [0, {L}]")
            valid = valid.to(device)
        return valid.contiguous()
    if valid.dim() != 2 or tuple(valid.shape) != (B, L):
        raise ValueError(f"valid must be int32 lengths [{B}] or a 0/1 mask [{B}, {L}]")
    m = valid.detach().to("cpu", torch.float32)
    if not bool(((m == 0) | (m == 1)).all()):
        raise ValueError("valid mask must hold only 0 and 1")
    lengths = m.sum(1).to(torch.int32)
    expect = (torch.arange(L)[None, :] < lengths[:, None]).to(torch.float32)
    if not torch.equal(expect, m):
        raise ValueError("valid mask must be right-padded: 1 on tokens, then 0 on pads")
    return lengths.to(device)


def _inputs(q, k, v, g, beta, valid, s0, s0_row):
    """Validate the torch arguments shared by prefill and decode; returns what the call needs."""
    import torch
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4:
        raise ValueError("q, k must be [B, L, Hk, D] and v [B, L, Hv, Dv]")
    B, L, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on the GPU")
    if q.dtype not in (torch.float32, torch.bfloat16) or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one dtype, float32 or bfloat16")
    if tuple(v.shape[:2]) != (B, L) or g.shape != (B, L, Hv) or beta.shape != (B, L, Hv):
        raise ValueError("v [B, L, Hv, Dv], g and beta [B, L, Hv] expected")
    if g.dtype != torch.float32:
        raise ValueError("g must be float32")
    if beta.dtype not in (torch.float32, q.dtype):
        raise ValueError("beta must be float32 or q's dtype")
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("s0", s0)):
        if t is not None and (t.device != dev or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous tensor on {dev}")
    lengths = _lengths_from_valid(valid, B, L, dev)
    n_s0 = 0
    if s0 is not None:
        if s0.dtype != torch.float32 or s0.dim() != 4 or tuple(s0.shape[1:]) != (Hv, Dk, Dv):
            raise ValueError(f"s0 must be float32 [n_s0, {Hv}, {Dk}, {Dv}]")
        n_s0 = s0.shape[0]
    if s0_row is not None:
        if s0 is None:
            raise ValueError("s0_row needs s0")
        if s0_row.dtype != torch.int32 or tuple(s0_row.shape) != (B,):
            raise ValueError(f"s0_row must be int32 [{B}]")
        if s0_row.device.type == "cpu":
            if B and (int(s0_row.min()) < 0 or int(s0_row.max()) >= n_s0):
                raise ValueError(f"s0_row entries must lie in [0, {n_s0})")
            s0_row = s0_row.to(dev)
        s0_row = s0_row.contiguous()
    desc = make_desc(B, L, Hk, Hv, n_s0, q.dtype == torch.bfloat16, beta.dtype == torch.bfloat16, Dk, Dv)
    return desc, lengths, s0_row, (B, L, Hk, Hv, Dk, Dv), dev


def prefill(q, k, v, g, beta, valid=None, s0=None, s0_row=None, *, want_state=True, out=None,
            s_final=None, workspace=None):
    """Run the chunked gated delta rule on torch's current stream; see the module docstring.

    out / s_final / workspace may be given to reuse buffers (s_final may be s0 itself, for an
    in-place continuation, when s0_row is None).
    """
    import torch
    desc, lengths, s0_row, (B, L, Hk, Hv, Dk, Dv), dev = _inputs(q, k, v, g, beta, valid, s0, s0_row)
    need = workspace_size(desc)
    o = out if out is not None else torch.empty(B, L, Hv, Dv, device=dev, dtype=v.dtype)
    if want_state and s_final is None:
        s_final = torch.empty(B, Hv, Dk, Dv, device=dev, dtype=torch.float32)
    if not want_state:
        s_final = None
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), device=dev, dtype=torch.uint8)
    stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        st = library().gdr_prefill(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                   _ptr(lengths), _ptr(s0), _ptr(s0_row), _ptr(o), _ptr(s_final),
                                   _ptr(workspace), need, stream)
    _raise(st)
    return o, s_final


def decode(q, k, v, g, beta, valid=None, s0=None, s0_row=None, *, want_state=True, out=None, s_final=None):
    """The same recurrence token by token (gdr_decode): for short sequences over many rows, with
    the same arguments and results as prefill and no workspace."""
    import torch
    desc, lengths, s0_row, (B, L, Hk, Hv, Dk, Dv), dev = _inputs(q, k, v, g, beta, valid, s0, s0_row)
    o = out if out is not None else torch.empty(B, L, Hv, Dv, device=dev, dtype=v.dtype)
    if want_state and s_final is None:
        s_final = torch.empty(B, Hv, Dk, Dv, device=dev, dtype=torch.float32)
    if not want_state:
        s_final = None
    stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        st = library().gdr_decode(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                  _ptr(lengths), _ptr(s0), _ptr(s0_row), _ptr(o), _ptr(s_final), stream)
    _raise(st)
    return o, s_final
