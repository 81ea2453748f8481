"""The C ABI on the CPU: the library loads, exports every declared symbol, sizes its
workspace, and rejects every invalid argument on the host before touching a GPU.

No compute call is made here: gdr_prefill is only called with arguments that fail host
validation (it returns before any HIP call), and valid argument sets go to the host-only
gdr_prefill_check. The pointers are fake integers; nothing dereferences them.
"""
import ctypes
import os
import re

import pytest

import gated_deltanet_prefill_gdr_amd as gdr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, EINVAL, EUNSUP, EWS = 0, -1, -2, -3


def header_functions():
    text = open(os.path.join(ROOT, "include", "gdr.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdr_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = gdr.library()
    names = header_functions()
    assert "gdr_prefill" in names and "gdr_prefill_check" in names and len(names) >= 7
    for n in names:
        assert hasattr(lib, n), n


def test_kernel_names():
    assert [gdr.kernel_name(i) for i in range(2)] == ["gdr_prep", "gdr_scan"]
    assert [gdr.kernel_name(i) for i in range(len(gdr.KERNELS))] == list(gdr.KERNELS)
    assert gdr.kernel_name(len(gdr.KERNELS)) == "" and gdr.kernel_name(-1) == ""


BASE = 1 << 32   # fake, 256-byte aligned device addresses, far apart


class Call:
    """A valid argument set (fake pointers) that single fields can be broken in."""

    def __init__(self, B=2, L=130, Hk=2, Hv=4, bf16=True, s0=True, s0_row=False, lengths=True, s_final=True):
        self.desc = gdr.make_desc(B, L, Hk, Hv, n_s0=B if s0 else 0, qkv_bf16=bf16)
        esz = 2 if bf16 else 4
        sizes = {"q": B * L * Hk * 128 * esz, "k": B * L * Hk * 128 * esz, "v": B * L * Hv * 128 * esz,
                 "g": B * L * Hv * 4, "beta": B * L * Hv * 4, "lengths": B * 4, "s0": B * Hv * 128 * 128 * 4,
                 "s0_row": B * 4, "o": B * L * Hv * 128 * esz, "s_final": B * Hv * 128 * 128 * 4}
        addr = BASE
        self.p = {}
        for name in ("q", "k", "v", "g", "beta", "lengths", "s0", "s0_row", "o", "s_final"):
            self.p[name] = addr
            addr += (sizes[name] + 4095) // 4096 * 4096 + 4096
        if not s0:
            self.p["s0"] = 0
        if not s0_row:
            self.p["s0_row"] = 0
        if not lengths:
            self.p["lengths"] = 0
        if not s_final:
            self.p["s_final"] = 0
        self.ws_bytes = gdr.workspace_size(self.desc)
        self.p["ws"] = addr

    def ptrs(self):
        return [self.p[n] for n in ("q", "k", "v", "g", "beta", "lengths", "s0", "s0_row", "o", "s_final", "ws")]

    def check(self):
        return gdr.check(self.desc, self.ptrs(), self.ws_bytes)

    def prefill(self):
        lib = gdr.library()
        return lib.gdr_prefill(ctypes.byref(self.desc), *[x or None for x in self.ptrs()], self.ws_bytes, None)


def test_valid_calls_pass_host_check():
    for kw in ({}, {"bf16": False}, {"s0": False}, {"s0_row": True}, {"lengths": False, "s_final": False}):
        assert Call(**kw).check() == OK, (kw, gdr.last_error())


def test_workspace_size():
    # one record per (row, value head, chunk): the 6 lower-triangle operand blocks (64 lanes x 8)
    # of the chunk's T diag(beta) (and, for float32, of its decayed causal scores), in q's dtype,
    # plus 8 x 64 floats of per-token scalars
    rec_bf16 = 6 * 512 * 2 + 8 * 64 * 4
    rec_f32 = 2 * 6 * 512 * 4 + 8 * 64 * 4
    assert rec_bf16 == 8192 and rec_f32 == 26624
    # bf16 sequences are cut into P segments scanned in parallel (P = ceil(256 / (B Hv)) capped
    # by the chunk count, then trimmed so no segment is empty), each with a 128 x 256 fp32 slot
    slot = 128 * 256 * 4
    # bf16 also keeps a list of the chunks that hold valid tokens (used when lengths are given):
    # an int32 count and one int32 per (row, chunk)
    lst = lambda B, NC: 4 * (1 + B * NC + B)   # chunk list, then the row order
    # with segments, a 256-byte-aligned tail: a 256-byte status header, then per (row, head, segment)
    # a 16-byte truncation plan entry and 16 floats of certificate parts
    up = lambda x: (x + 255) // 256 * 256
    tail = lambda n: 256 + n * (16 + 64)
    base = 32 * 256 * rec_bf16 + 32 * 8 * slot + lst(1, 256)
    assert gdr.workspace_size(gdr.make_desc(1, 16384, 16, 32, qkv_bf16=True)) == up(base) + tail(32 * 8)
    base = 2 * 4 * rec_bf16 + 2 * 4 * slot + lst(1, 4)
    assert gdr.workspace_size(gdr.make_desc(1, 200, 1, 2, qkv_bf16=True)) == up(base) + tail(2 * 4)
    base = 100 * 10 * rec_bf16 + 100 * 3 * slot + lst(1, 10)
    assert gdr.workspace_size(gdr.make_desc(1, 640, 2, 100, qkv_bf16=True)) == up(base) + tail(100 * 3)
    d = gdr.make_desc(1, 16384, 16, 32, qkv_bf16=True)
    assert gdr.status_offset(d) == up(32 * 256 * rec_bf16 + 32 * 8 * slot + lst(1, 256))
    assert gdr.status_offset(gdr.make_desc(64, 1024, 16, 32, qkv_bf16=True)) is None   # one segment
    assert gdr.workspace_size(gdr.make_desc(64, 1024, 16, 32, qkv_bf16=True)) == 64 * 32 * 16 * rec_bf16 + lst(64, 16)
    assert gdr.workspace_size(gdr.make_desc(2, 130, 2, 4)) == 2 * 4 * 3 * rec_f32
    assert gdr.workspace_size(gdr.make_desc(0, 100, 1, 1)) == 0
    assert gdr.workspace_size(gdr.make_desc(3, 0, 1, 1)) == 0
    # a partial chunk counts as a whole one
    assert gdr.workspace_size(gdr.make_desc(1, 65, 1, 1)) == gdr.workspace_size(gdr.make_desc(1, 128, 1, 1))
    with pytest.raises(gdr.GdrError):
        gdr.workspace_size(gdr.make_desc(1, 64, 3, 4))


def broken(mutate):
    c = Call()
    mutate(c)
    st_check = c.check()
    st_run = c.prefill()   # fails in host validation, before any HIP call
    assert st_check == st_run
    return st_check, gdr.last_error()


@pytest.mark.parametrize("field,value,status,msg", [
    ("B", -1, EINVAL, "must be >= 0"),
    ("L", -5, EINVAL, "must be >= 0"),
    ("Hk", 0, EINVAL, "must be > 0"),
    ("Hv", 3, EINVAL, "multiple of Hk"),
    ("Dk", 64, EUNSUP, "128"),
    ("Dv", 256, EUNSUP, "128"),
    ("qkv_dtype", 7, EINVAL, "not a gdr_dtype"),
    ("beta_dtype", 5, EINVAL, "beta_dtype"),
    ("n_s0", 0, EINVAL, "n_s0"),
    ("n_s0", 1, EINVAL, "n_s0"),
])
def test_desc_errors(field, value, status, msg):
    st, err = broken(lambda c: setattr(c.desc, field, value))
    assert st == status and msg in err


def test_size_limits():
    """Shapes past the launch-grid limits or the 32-bit buffer offsets of one batch row are refused on the
    host with GDR_EUNSUPPORTED (and the workspace query raises), before any launch; the longest row
    that fits is accepted."""
    cases = [({"B": 70000}, "grid limits"),                              # B > 65535
             ({"B": 40000, "L": 64 * 60000, "Hv": 2}, "grid limits"),    # B Hv ceil(L/64) >= 2^31
             ({"B": 1, "L": 1 << 18, "Hv": 32}, "4 GiB")]                # (L + 128) Hv 512 bytes >= 4 GiB
    for fields, msg in cases:
        c = Call(B=1, L=130, Hk=1, Hv=2, s0=False)
        for k, v in fields.items():
            setattr(c.desc, k, v)
        assert c.check() == EUNSUP and msg in gdr.last_error(), (fields, gdr.last_error())
        assert c.prefill() == EUNSUP
        with pytest.raises(gdr.GdrError, match=msg):
            gdr.workspace_size(c.desc)
    c = Call(B=1, L=(1 << 18) - 256, Hk=1, Hv=32, s0=False)   # (L + 128) Hv 512 bytes just below 4 GiB
    assert c.check() == OK, gdr.last_error()


def test_beta_dtype_mismatch():
    def m(c):
        c.desc.qkv_dtype = gdr.GDR_F32
        c.desc.beta_dtype = gdr.GDR_BF16
        c.ws_bytes = gdr.workspace_size(gdr.make_desc(2, 130, 2, 4, n_s0=2))
    st, err = broken(m)
    assert st == EINVAL and "beta_dtype" in err


@pytest.mark.parametrize("name", ["q", "k", "v", "g", "beta", "o"])
def test_null_required_pointer(name):
    st, err = broken(lambda c: c.p.__setitem__(name, 0))
    assert st == EINVAL and "non-NULL" in err


@pytest.mark.parametrize("name", ["q", "k", "v", "o", "s0", "s_final"])
def test_misaligned_pointer(name):
    st, err = broken(lambda c: c.p.__setitem__(name, c.p[name] + 8))
    assert st == EINVAL and "aligned" in err


def test_misaligned_workspace():
    st, err = broken(lambda c: c.p.__setitem__("ws", c.p["ws"] + 16))
    assert st == EINVAL and "workspace" in err


def test_workspace_missing_or_small():
    st, err = broken(lambda c: c.p.__setitem__("ws", 0))
    assert st == EWS and "NULL" in err
    st, err = broken(lambda c: setattr(c, "ws_bytes", c.ws_bytes - 1))
    assert st == EWS and "needed" in err


def test_s0_row_without_s0():
    def m(c):
        c.p["s0"] = 0
        c.p["s0_row"] = c.p["lengths"] + 1024
    st, err = broken(m)
    assert st == EINVAL and "s0_row" in err


def test_in_place_state():
    c = Call()
    c.p["s_final"] = c.p["s0"]
    assert c.check() == OK                      # in place without s0_row: allowed
    c.p["s0_row"] = c.p["lengths"] + 4096
    assert c.check() == EINVAL and "alias" in gdr.last_error()


@pytest.mark.parametrize("out,inp", [("o", "q"), ("o", "v"), ("s_final", "k"), ("ws", "g"), ("o", "s0"),
                                     ("s_final", "beta")])
def test_outputs_must_not_overlap_inputs(out, inp):
    st, err = broken(lambda c: c.p.__setitem__(out, c.p[inp] + 256))
    assert st == EINVAL and "overlaps" in err


def test_outputs_must_not_overlap_each_other():
    st, err = broken(lambda c: c.p.__setitem__("s_final", c.p["o"] + 4096))
    assert st == EINVAL and "overlaps" in err


def test_empty_problems_need_no_pointers():
    for B, L in ((0, 100), (3, 0)):
        d = gdr.make_desc(B, L, 1, 2)
        assert gdr.check(d, [0] * 11, 0) == OK


def decode_call(c):
    lib = gdr.library()
    return lib.gdr_decode(ctypes.byref(c.desc), *[x or None for x in c.ptrs()[:10]], None)


@pytest.mark.parametrize("mutate,status,msg", [
    (lambda c: c.p.__setitem__("q", 0), EINVAL, "non-NULL"),
    (lambda c: c.p.__setitem__("v", c.p["v"] + 8), EINVAL, "aligned"),
    (lambda c: c.p.__setitem__("o", c.p["k"] + 256), EINVAL, "overlaps"),
    (lambda c: (c.p.__setitem__("s_final", c.p["s0"]), c.p.__setitem__("s0_row", c.p["lengths"] + 4096)),
     EINVAL, "alias"),
    (lambda c: setattr(c.desc, "Dk", 64), EUNSUP, "Dk"),
])
def test_decode_rejects_invalid_arguments_on_host(mutate, status, msg):
    """gdr_decode runs gdr_prefill's host validation (minus the workspace) before any launch."""
    c = Call()
    mutate(c)
    assert decode_call(c) == status
    assert msg in gdr.last_error()


def test_decode_empty_problems_need_no_pointers():
    lib = gdr.library()
    for B, L in ((0, 5), (3, 0)):
        d = gdr.make_desc(B, L, 1, 2)
        assert lib.gdr_decode(ctypes.byref(d), *[None] * 10, None) == OK


# ---------------------------------------------------------------- layer steps
def test_gates_host_validation():
    lib = gdr.library()
    P = [BASE + i * (1 << 20) for i in range(7)]
    ok = lambda *ptrs: lib.gdr_gates(2, 5, 4, 1, *ptrs, None)
    assert lib.gdr_gates(0, 5, 4, 1, *[None] * 7, None) == OK          # empty: no pointers needed
    assert lib.gdr_gates(2, 5, 0, 1, *[None] * 7, None) == EINVAL and "Hv" in gdr.last_error()
    assert lib.gdr_gates(2, 5, 4, 7, *P, None) == EINVAL and "dtype" in gdr.last_error()
    assert ok(None, *P[1:]) == EINVAL and "non-NULL" in gdr.last_error()
    assert ok(P[0] + 1, *P[1:]) == EINVAL and "aligned" in gdr.last_error()
    bad = list(P)
    bad[5] = P[0] + 4                                                   # beta over b
    assert ok(*bad) == EINVAL and "overlaps" in gdr.last_error()


def test_conv_silu_host_validation():
    lib = gdr.library()
    P = [BASE + i * (1 << 24) for i in range(8)]   # mixed tail w lengths q k v new_tail
    call = lambda K, ptrs, B=2, L=10, dt=1: lib.gdr_conv_silu(B, L, 1, 2, K, dt, *ptrs, None)
    assert call(0, P) == EUNSUP and "K" in gdr.last_error()
    assert call(9, P) == EUNSUP
    assert call(4, P, B=0) == OK and call(4, [None] * 8, B=0) == OK
    assert call(4, [None] * 8, L=0) == OK                               # nothing to compute or carry
    assert call(4, [None] * 7 + [P[7]], L=0) == EINVAL and "w" in gdr.last_error()   # a tail to carry needs w
    bad = list(P)
    bad[4] = P[0] + 64                                                  # q over mixed
    assert call(4, bad) == EINVAL and "overlaps" in gdr.last_error()
    bad = list(P)
    bad[7] = P[1] + 16                                                  # new_tail partly over tail (not in place)
    assert call(4, bad) == EINVAL and "overlaps" in gdr.last_error()
    bad = list(P)
    bad[0] = P[0] + 8
    assert call(4, bad) == EINVAL and "aligned" in gdr.last_error()
    assert lib.gdr_conv_silu(2, 64 * 65536, 1, 2, 4, 1, *P, None) == EUNSUP


def test_gated_rmsnorm_host_validation():
    lib = gdr.library()
    f = ctypes.c_float
    P = [BASE + i * (1 << 24) for i in range(4)]   # x z w out
    call = lambda rows, ptrs, eps=1e-6, dt=1: lib.gdr_gated_rmsnorm(rows, dt, ptrs[0], ptrs[1], ptrs[2], f(eps), ptrs[3], None)
    assert call(0, [None] * 4) == OK
    assert call(-1, P) == EINVAL
    assert call(8, P, eps=-1.0) == EINVAL and "eps" in gdr.last_error()
    assert call(8, P, eps=float("nan")) == EINVAL
    assert call(8, [P[0], P[1], P[2], P[1]]) == EINVAL and "overlaps" in gdr.last_error()   # out over z
    assert call(8, [P[0] + 8, P[1], P[2], P[3]]) == EINVAL and "aligned" in gdr.last_error()
    assert call(8, [None, P[1], P[2], P[3]]) == EINVAL and "non-NULL" in gdr.last_error()


# ---------------------------------------------------------------- gdr_prefill_ex (fused gates / norm)
def prefill_ex(c, fu, g_beta=True):
    lib = gdr.library()
    ptrs = [x or None for x in c.ptrs()]
    if not g_beta:
        ptrs[3] = ptrs[4] = None
    return lib.gdr_prefill_ex(ctypes.byref(c.desc), *ptrs[:8], ctypes.byref(fu), ptrs[8], ptrs[9], ptrs[10],
                              c.ws_bytes, None)


def fusion(c, gates=True, norm=True):
    fu = gdr.Fusion()
    base = c.p["ws"] + (1 << 30)
    if gates:
        fu.b_raw, fu.a_raw, fu.A_log, fu.dt_bias = base, base + (1 << 24), base + (2 << 24), base + (3 << 24)
    if norm:
        fu.z, fu.norm_w, fu.norm_eps = base + (4 << 24), base + (5 << 24), 1e-6
    return fu


@pytest.mark.parametrize("mutate,g_beta,msg", [
    (lambda f: None, True, "must be NULL"),                           # g, beta given with fused gates
    (lambda f: setattr(f, "A_log", None), False, "go together"),
    (lambda f: setattr(f, "norm_w", None), False, "go together"),
    (lambda f: setattr(f, "norm_eps", -1.0), False, "norm_eps"),
    (lambda f: setattr(f, "norm_eps", float("inf")), False, "norm_eps"),
    (lambda f: setattr(f, "norm_w", f.norm_w + 4), False, "aligned"),
    (lambda f: setattr(f, "b_raw", f.b_raw + 1), False, "aligned"),
])
def test_prefill_ex_rejects_bad_fusion(mutate, g_beta, msg):
    c = Call()
    fu = fusion(c)
    mutate(fu)
    assert prefill_ex(c, fu, g_beta) == EINVAL
    assert msg in gdr.last_error()


def test_prefill_ex_output_must_not_overlap_fused_inputs():
    c = Call()
    fu = fusion(c)
    fu.z = c.p["o"] + 256
    assert prefill_ex(c, fu, g_beta=False) == EINVAL and "overlaps z" in gdr.last_error()
    fu = fusion(c)
    fu.b_raw = c.p["s_final"]
    assert prefill_ex(c, fu, g_beta=False) == EINVAL and "overlaps b_raw" in gdr.last_error()


def test_prefill_ex_without_fused_gates_still_needs_g_and_beta():
    c = Call()
    fu = fusion(c, gates=False)
    assert prefill_ex(c, fu, g_beta=False) == EINVAL and "non-NULL" in gdr.last_error()


def test_decode_ex_validates_fusion_like_prefill_ex():
    c = Call()
    fu = fusion(c)
    lib = gdr.library()
    ptrs = [x or None for x in c.ptrs()]
    st = lib.gdr_decode_ex(ctypes.byref(c.desc), *ptrs[:8], ctypes.byref(fu), ptrs[8], ptrs[9], None)
    assert st == EINVAL and "must be NULL" in gdr.last_error()      # g, beta given with fused gates
    fu.norm_eps = -1.0
    ptrs[3] = ptrs[4] = None
    st = lib.gdr_decode_ex(ctypes.byref(c.desc), *ptrs[:8], ctypes.byref(fu), ptrs[8], ptrs[9], None)
    assert st == EINVAL and "norm_eps" in gdr.last_error()


# ---------------------------------------------------------------- caller-supplied outputs (binding)
def test_binding_rejects_bad_output_buffers():
    """The binding checks every caller-supplied output like the inputs: the C ABI sizes writes from
    the descriptor and cannot see the real allocation (CPU tensors stand in for device ones here)."""
    import torch
    cpu = torch.device("cpu")
    ok = torch.empty(2, 3, 4, 128, dtype=torch.bfloat16)
    gdr.check_buffer("out", ok, (2, 3, 4, 128), torch.bfloat16, cpu)
    bad = {
        "short": torch.empty(2, 3, 3, 128, dtype=torch.bfloat16),
        "dtype": torch.empty(2, 3, 4, 128, dtype=torch.float32),
        "strided": torch.empty(2, 3, 128, 4, dtype=torch.bfloat16).transpose(2, 3),
    }
    for why, t in bad.items():
        with pytest.raises(ValueError):
            gdr.check_buffer("out", t, (2, 3, 4, 128), torch.bfloat16, cpu)
    with pytest.raises(ValueError):   # another device
        gdr.check_buffer("out", ok, (2, 3, 4, 128), torch.bfloat16, torch.device("cuda", 0))
    gdr.check_workspace(torch.empty(100, dtype=torch.uint8), 100, cpu)
    for ws in (torch.empty(99, dtype=torch.uint8), torch.empty(25, dtype=torch.float32),
               torch.empty(200, dtype=torch.uint8)[::2], torch.empty(10, 10, dtype=torch.uint8)):
        with pytest.raises(ValueError):
            gdr.check_workspace(ws, 100, cpu)
