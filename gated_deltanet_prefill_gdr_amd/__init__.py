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

__all__ = ["prefill", "prefill_noalloc", "workspace_size", "check", "last_error", "library", "timing_enable", "set_truncation",
           "status_offset",
           "timing_read", "kernel_name", "GdrError", "KERNELS", "LIB_PATH", "decode", "gates", "conv_silu",
           "gated_rmsnorm"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdr.so")
HEAD_DIM = 128
GDR_F32, GDR_BF16 = 0, 1
STATUS = {0: "GDR_OK", -1: "GDR_EINVAL", -2: "GDR_EUNSUPPORTED", -3: "GDR_EWORKSPACE", -4: "GDR_EHIP"}
KERNELS = ("gdr_prep", "gdr_scan", "gdr_transition", "gdr_combine", "gdr_decode", "gdr_gates", "gdr_conv_silu",
           "gdr_gated_rmsnorm", "gdr_finalize")


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
    lib.gdr_prefill_ex.argtypes = [ctypes.POINTER(Desc)] + [vp] * 8 + [ctypes.POINTER(Fusion)] + [vp] * 3 + [sz, vp]
    lib.gdr_prefill_ex.restype = i32
    lib.gdr_prefill_noalloc.argtypes = [ctypes.POINTER(Desc)] + [vp] * 10 + [vp]
    lib.gdr_prefill_noalloc.restype = i32
    lib.gdr_decode.argtypes = [ctypes.POINTER(Desc)] + [vp] * 10 + [vp]
    lib.gdr_decode_ex.argtypes = [ctypes.POINTER(Desc)] + [vp] * 8 + [ctypes.POINTER(Fusion)] + [vp] * 2 + [vp]
    lib.gdr_decode_ex.restype = i32
    lib.gdr_decode.restype = i32
    i64, f32 = ctypes.c_int64, ctypes.c_float
    lib.gdr_gates.argtypes = [i32, i32, i32, i32] + [vp] * 7 + [vp]
    lib.gdr_gates.restype = i32
    lib.gdr_conv_silu.argtypes = [i32, i32, i32, i32, i32, i32] + [vp] * 8 + [vp]
    lib.gdr_conv_silu.restype = i32
    lib.gdr_gated_rmsnorm.argtypes = [i64, i32, vp, vp, vp, f32, vp, vp]
    lib.gdr_gated_rmsnorm.restype = i32
    lib.gdr_last_error.argtypes = []
    lib.gdr_last_error.restype = ctypes.c_char_p
    lib.gdr_timing_enable.argtypes = [i32]
    lib.gdr_timing_enable.restype = i32
    lib.gdr_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64), i32]
    lib.gdr_timing_read.restype = i32
    lib.gdr_kernel_name.argtypes = [i32]
    lib.gdr_kernel_name.restype = ctypes.c_char_p
    lib.gdr_set_truncation.argtypes = [i32]
    lib.gdr_set_truncation.restype = i32
    lib.gdr_prefill_status_offset.argtypes = [ctypes.POINTER(Desc)]
    lib.gdr_prefill_status_offset.restype = sz
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


def set_truncation(on: bool = True):
    """Allow (default) or forbid truncated segment starts for every later call (gdr_set_truncation)."""
    _raise(library().gdr_set_truncation(1 if on else 0))


def status_offset(desc: Desc):
    """Byte offset of the status word (heads rerun without truncation) in the workspace, or None when the
    shape has no segments."""
    n = library().gdr_prefill_status_offset(ctypes.byref(desc))
    return None if n == ctypes.c_size_t(-1).value else n


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


def _inputs(q, k, v, g, beta, valid, s0, s0_row, gates=None):
    """Validate the torch arguments shared by prefill and decode; returns what the call needs.

    With ``gates`` = (b_raw, a_raw, A_log, dt_bias) given, g and beta must be None and the raw
    projections set the beta dtype."""
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
    if tuple(v.shape[:2]) != (B, L):
        raise ValueError("v [B, L, Hv, Dv] expected")
    if gates is not None:
        if g is not None or beta is not None:
            raise ValueError("g and beta must be None when the gate prologue is fused")
        b_raw, a_raw, A_log, dt_bias = gates
        if b_raw.shape != (B, L, Hv) or a_raw.shape != (B, L, Hv) or a_raw.dtype != b_raw.dtype:
            raise ValueError("b_raw and a_raw must be [B, L, Hv] of one dtype")
        if b_raw.dtype not in (torch.float32, q.dtype):
            raise ValueError("b_raw must be float32 or q's dtype")
        if A_log.shape != (Hv,) or dt_bias.shape != (Hv,) or A_log.dtype != torch.float32 or dt_bias.dtype != torch.float32:
            raise ValueError(f"A_log and dt_bias must be float32 [{Hv}]")
        beta_dtype = b_raw.dtype
        extra = (("b_raw", b_raw), ("a_raw", a_raw), ("A_log", A_log), ("dt_bias", dt_bias))
    else:
        if g is None or beta is None or g.shape != (B, L, Hv) or beta.shape != (B, L, Hv):
            raise ValueError("g and beta [B, L, Hv] expected")
        if g.dtype != torch.float32:
            raise ValueError("g must be float32")
        if beta.dtype not in (torch.float32, q.dtype):
            raise ValueError("beta must be float32 or q's dtype")
        beta_dtype = beta.dtype
        extra = ()
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("s0", s0)) + extra:
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
    desc = make_desc(B, L, Hk, Hv, n_s0, q.dtype == torch.bfloat16, beta_dtype == torch.bfloat16, Dk, Dv)
    return desc, lengths, s0_row, (B, L, Hk, Hv, Dk, Dv), dev


class Fusion(ctypes.Structure):
    _fields_ = [("b_raw", ctypes.c_void_p), ("a_raw", ctypes.c_void_p), ("A_log", ctypes.c_void_p),
                ("dt_bias", ctypes.c_void_p), ("z", ctypes.c_void_p), ("norm_w", ctypes.c_void_p),
                ("norm_eps", ctypes.c_float)]


def _fusion(gates, norm, v, dev):
    """The gdr_fusion struct for gates = (b_raw, a_raw, A_log, dt_bias) and norm = (z, norm_w, eps),
    or None when neither is given (the gate tensors are checked by _inputs)."""
    import torch
    if gates is None and norm is None:
        return None
    fu = Fusion()
    if gates is not None:
        fu.b_raw, fu.a_raw, fu.A_log, fu.dt_bias = (t.data_ptr() for t in gates)
    if norm is not None:
        z, nw, eps = norm
        if z.shape != v.shape or z.dtype != v.dtype or nw.shape != (v.shape[3],) or nw.dtype != torch.float32:
            raise ValueError("norm: z must match v's shape and dtype and norm_w be float32 [128]")
        for name, t in (("z", z), ("norm_w", nw)):
            if t.device != dev or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous tensor on {dev}")
        fu.z, fu.norm_w, fu.norm_eps = z.data_ptr(), nw.data_ptr(), float(eps)
    return fu


def prefill(q, k, v, g, beta, valid=None, s0=None, s0_row=None, *, gates=None, norm=None, want_state=True,
            out=None, s_final=None, workspace=None):
    """Run the chunked gated delta rule on torch's current stream; see the module docstring.

    out / s_final / workspace may be given to reuse buffers (s_final may be s0 itself, for an
    in-place continuation, when s0_row is None).

    Fused work (gdr_prefill_ex): ``gates`` = (b_raw, a_raw, A_log, dt_bias) forms beta and g from
    the raw projections inside the kernels (pass g = beta = None); ``norm`` = (z, norm_w, eps)
    returns the gated RMSNorm w o / rms(o) silu(z) of the output instead of o.
    """
    import torch
    desc, lengths, s0_row, (B, L, Hk, Hv, Dk, Dv), dev = _inputs(q, k, v, g, beta, valid, s0, s0_row, gates)
    fu = _fusion(gates, norm, v, dev)
    need = workspace_size(desc)
    if out is not None:
        check_buffer("out", out, (B, L, Hv, Dv), v.dtype, dev)
    o = out if out is not None else torch.empty(B, L, Hv, Dv, device=dev, dtype=v.dtype)
    if s_final is not None:
        check_buffer("s_final", s_final, (B, Hv, Dk, Dv), torch.float32, dev)
    if want_state and s_final is None:
        s_final = torch.empty(B, Hv, Dk, Dv, device=dev, dtype=torch.float32)
    if not want_state:
        s_final = None
    if workspace is not None:
        check_workspace(workspace, need, dev)
    else:
        workspace = torch.empty(max(need, 1), device=dev, dtype=torch.uint8)
    stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        st = library().gdr_prefill_ex(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                      _ptr(lengths), _ptr(s0), _ptr(s0_row), None if fu is None else ctypes.byref(fu),
                                      _ptr(o), _ptr(s_final), _ptr(workspace), need, stream)
    _raise(st)
    return o, s_final


def prefill_noalloc(q, k, v, g, beta, valid=None, s0=None, s0_row=None, *, out, s_final=None):
    """gdr_prefill_noalloc: the prefill with the library's device-resident workspace (no workspace
    argument; shapes needing more than 128 MiB of workspace are rejected). The outputs are the
    caller's: out [B, L, Hv, 128] in v's dtype and s_final [B, Hv, 128, 128] float32 (or None)."""
    import torch
    desc, lengths, s0_row, (B, L, Hk, Hv, Dk, Dv), dev = _inputs(q, k, v, g, beta, valid, s0, s0_row)
    check_buffer("out", out, (B, L, Hv, Dv), v.dtype, dev)
    if s_final is not None:
        check_buffer("s_final", s_final, (B, Hv, Dk, Dv), torch.float32, dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        st = library().gdr_prefill_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                           _ptr(lengths), _ptr(s0), _ptr(s0_row), _ptr(out), _ptr(s_final), stream)
    _raise(st)
    return out, s_final


def decode(q, k, v, g, beta, valid=None, s0=None, s0_row=None, *, gates=None, norm=None, want_state=True, out=None,
           s_final=None):
    """The same recurrence token by token (gdr_decode_ex): for short sequences over many rows, with
    the same arguments (fused gates / norm included) and results as prefill and no workspace."""
    import torch
    desc, lengths, s0_row, (B, L, Hk, Hv, Dk, Dv), dev = _inputs(q, k, v, g, beta, valid, s0, s0_row, gates)
    fu = _fusion(gates, norm, v, dev)
    if out is not None:
        check_buffer("out", out, (B, L, Hv, Dv), v.dtype, dev)
    o = out if out is not None else torch.empty(B, L, Hv, Dv, device=dev, dtype=v.dtype)
    if s_final is not None:
        check_buffer("s_final", s_final, (B, Hv, Dk, Dv), torch.float32, dev)
    if want_state and s_final is None:
        s_final = torch.empty(B, Hv, Dk, Dv, device=dev, dtype=torch.float32)
    if not want_state:
        s_final = None
    stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        st = library().gdr_decode_ex(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                     _ptr(lengths), _ptr(s0), _ptr(s0_row), None if fu is None else ctypes.byref(fu),
                                     _ptr(o), _ptr(s_final), stream)
    _raise(st)
    return o, s_final


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return GDR_BF16
    if t.dtype == torch.float32:
        return GDR_F32
    raise ValueError("tensors must be float32 or bfloat16")


def check_buffer(name, t, shape, dtype, dev):
    """A caller-supplied output buffer must be exactly what the kernels write: the C ABI sizes every
    range from the descriptor and cannot see the real allocation, so a short, mistyped, strided or
    foreign buffer would be written out of bounds. Raises ValueError otherwise."""
    shape = tuple(int(x) for x in shape)
    if tuple(t.shape) != shape or t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} {list(shape)}, got {t.dtype} {list(t.shape)}")
    if t.device != dev or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous tensor on {dev}")


def check_workspace(ws, need, dev):
    """The workspace must be a contiguous uint8 tensor on the call's device with at least `need` bytes."""
    import torch
    if ws.dtype != torch.uint8 or ws.dim() != 1 or ws.device != dev or not ws.is_contiguous():
        raise ValueError(f"workspace must be a contiguous 1-D uint8 tensor on {dev}")
    if ws.numel() < need:
        raise ValueError(f"workspace has {ws.numel()} bytes, {need} needed")


def _on(dev, **tensors):
    for name, t in tensors.items():
        if t is not None and (t.device != dev or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous tensor on {dev}")


def gates(b, a, A_log, dt_bias, valid=None, *, beta_out=None, g_out=None):
    """Gate prologue (gdr_gates): beta = sigmoid(b) [valid], g = -exp(A_log) softplus(a + dt_bias) [valid].

    b, a [B, L, Hv] float32 or bfloat16 (same dtype); A_log, dt_bias [Hv] float32. Returns
    beta [B, L, Hv] in b's dtype and g [B, L, Hv] float32."""
    import torch
    if b.dim() != 3 or a.shape != b.shape or a.dtype != b.dtype:
        raise ValueError("b and a must be [B, L, Hv] of one dtype")
    B, L, Hv = b.shape
    dev = b.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on the GPU")
    code = _dtype_code(b)
    if A_log.shape != (Hv,) or dt_bias.shape != (Hv,) or A_log.dtype != torch.float32 or dt_bias.dtype != torch.float32:
        raise ValueError(f"A_log and dt_bias must be float32 [{Hv}]")
    _on(dev, b=b, a=a, A_log=A_log, dt_bias=dt_bias)
    lengths = _lengths_from_valid(valid, B, L, dev)
    if beta_out is not None:
        check_buffer("beta_out", beta_out, (B, L, Hv), b.dtype, dev)
    if g_out is not None:
        check_buffer("g_out", g_out, (B, L, Hv), torch.float32, dev)
    beta = beta_out if beta_out is not None else torch.empty_like(b)
    g = g_out if g_out is not None else torch.empty(B, L, Hv, device=dev, dtype=torch.float32)
    stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        st = library().gdr_gates(B, L, Hv, code, _ptr(b), _ptr(a), _ptr(A_log), _ptr(dt_bias), _ptr(lengths),
                                 _ptr(beta), _ptr(g), stream)
    _raise(st)
    return beta, g


def conv_silu(mixed, w, Hk, Hv, tail=None, valid=None, *, want_tail=True, new_tail=None, out=None):
    """Causal depthwise conv + SiLU with tail continuation and the q/k/v split (gdr_conv_silu).

    mixed [B, L, (2 Hk + Hv) 128] float32 or bfloat16; w [Cm, K] float32; tail [B, K-1, Cm] in
    mixed's dtype or None (zeros). Returns q [B, L, Hk, 128], k [B, L, Hk, 128], v [B, L, Hv, 128]
    and new_tail [B, K-1, Cm] (None if not wanted; pass new_tail=tail to update it in place)."""
    import torch
    if mixed.dim() != 3:
        raise ValueError("mixed must be [B, L, Cm]")
    B, L, Cm = mixed.shape
    if Cm != (2 * Hk + Hv) * HEAD_DIM:
        raise ValueError(f"mixed has {Cm} channels, (2 Hk + Hv) * 128 = {(2 * Hk + Hv) * HEAD_DIM} expected")
    dev = mixed.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on the GPU")
    code = _dtype_code(mixed)
    if w.dim() != 2 or w.shape[0] != Cm or w.dtype != torch.float32:
        raise ValueError(f"w must be float32 [{Cm}, K]")
    K = w.shape[1]
    if tail is not None and (tail.shape != (B, K - 1, Cm) or tail.dtype != mixed.dtype):
        raise ValueError(f"tail must be [{B}, {K - 1}, {Cm}] in mixed's dtype")
    _on(dev, mixed=mixed, w=w, tail=tail)
    if new_tail is not None:
        check_buffer("new_tail", new_tail, (B, K - 1, Cm), mixed.dtype, dev)
    lengths = _lengths_from_valid(valid, B, L, dev)
    if out is not None:
        if len(out) != 3:
            raise ValueError("out must be a tuple (q, k, v)")
        for name, t, H in (("q", out[0], Hk), ("k", out[1], Hk), ("v", out[2], Hv)):
            check_buffer(f"out {name}", t, (B, L, H, HEAD_DIM), mixed.dtype, dev)
    if out is None:
        q = torch.empty(B, L, Hk, HEAD_DIM, device=dev, dtype=mixed.dtype)
        k = torch.empty_like(q)
        v = torch.empty(B, L, Hv, HEAD_DIM, device=dev, dtype=mixed.dtype)
    else:
        q, k, v = out
    if want_tail and new_tail is None:
        new_tail = torch.empty(B, K - 1, Cm, device=dev, dtype=mixed.dtype)
    if not want_tail:
        new_tail = None
    stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        st = library().gdr_conv_silu(B, L, Hk, Hv, K, code, _ptr(mixed), _ptr(tail), _ptr(w), _ptr(lengths),
                                     _ptr(q), _ptr(k), _ptr(v), _ptr(new_tail), stream)
    _raise(st)
    return q, k, v, new_tail


def gated_rmsnorm(x, z, w, eps, *, out=None):
    """Gated RMSNorm over the last axis (128): w x / sqrt(mean(x^2) + eps) silu(z) (gdr_gated_rmsnorm).

    x, z [..., 128] of one dtype (float32 or bfloat16); w [128] float32. out may be x (in place)."""
    import torch
    if x.shape != z.shape or x.dtype != z.dtype or x.shape[-1] != HEAD_DIM:
        raise ValueError("x and z must share shape [..., 128] and dtype")
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on the GPU")
    code = _dtype_code(x)
    if w.shape != (HEAD_DIM,) or w.dtype != torch.float32:
        raise ValueError("w must be float32 [128]")
    _on(dev, x=x, z=z, w=w)
    if out is not None:
        check_buffer("out", out, tuple(x.shape), x.dtype, dev)
    y = out if out is not None else torch.empty_like(x)
    stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        st = library().gdr_gated_rmsnorm(x.numel() // HEAD_DIM, code, _ptr(x), _ptr(z), _ptr(w), float(eps), _ptr(y),
                                         stream)
    _raise(st)
    return y
