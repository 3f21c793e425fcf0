"""The C-ABI library on the CPU: it loads, exports every function the header
declares, and validates arguments (status codes, nothing launched) without a
GPU. Mirrors the asserts of the page's host_args / mla_post as negative tests.
"""

from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest
import torch

import mla_split_kv_amd as m

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h"))

OK, EINVAL, ESTRIDE, EALIGN, ERANGE, EUNSUP = 0, -1, -2, -3, -4, -5


def header_functions():
    """Every mla_* function the headers under include/ declare."""
    names = set()
    for h in HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(mla_\w+)\s*\(", src, flags=re.M))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    return m.load()


def test_header_declares_expected_entry_points():
    assert header_functions() == sorted(m.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", m.LIB_PATH], capture_output=True, text=True, check=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in header_functions():
        assert name in syms, f"{name} not exported"
        assert hasattr(lib, name)


def test_version_and_strerror(lib):
    assert lib.mla_post_version() == 5
    for st in (0, -1, -2, -3, -4, -5, -6):
        assert lib.mla_post_strerror(st).decode()
    assert lib.mla_post_strerror(-99).decode() == "unknown status"
    assert ctypes.sizeof(m.MlaPostArgs) == 224
    assert m.MlaPostArgs.q.offset == m.ARGS_V1_SIZE == 176


def good_args(n=4, S=8):
    """Valid arguments with fake (never dereferenced) device addresses."""
    a = m.MlaPostArgs()
    a.struct_size = ctypes.sizeof(m.MlaPostArgs)
    a.n, a.S = n, S
    a.o = 0x100000
    a.o_sj, a.o_st, a.o_sh = S * 6144, 6144, 512
    a.lse = 0x200000
    a.l_sj, a.l_st, a.l_sh = S * 12, 12, 1
    a.w_v = 0x300000
    a.w_sh, a.w_sv = 128 * 256, 256
    a.w_v_scale = 0x400000
    a.s_sh, a.s_sv, a.s_sb = 128 * 16, 16, 1
    a.gate = 0x500000
    a.core = 0x600000
    return a


def check(lib, a):
    return lib.mla_post_check(ctypes.byref(a))


def test_valid_args_pass(lib):
    assert check(lib, good_args()) == OK
    a = good_args(n=1)
    a.lse = None
    assert check(lib, a) == OK  # one partial, no LSE: the final attention output
    a = good_args(n=512, S=1)
    assert check(lib, a) == OK
    a = good_args(S=0)
    a.o = None  # empty batch: nothing is read
    assert check(lib, a) == OK


@pytest.mark.parametrize(
    "field,value,status",
    [
        ("struct_size", 8, EINVAL),
        ("n", 0, EINVAL),
        ("n", 513, EUNSUP),
        ("S", -1, EINVAL),
        ("o", None, EINVAL),
        ("lse", None, EINVAL),  # n > 1 needs LSEs
        ("w_v", None, EINVAL),
        ("w_v_scale", None, EINVAL),
        ("gate", None, EINVAL),
        ("core", None, EINVAL),
        ("o_sj", -6144, ESTRIDE),
        ("o_st", 6143, ESTRIDE),
        ("o_sh", 4, ESTRIDE),
        ("l_st", -1, ESTRIDE),
        ("w_sv", 255, ESTRIDE),
        ("w_sh", -256, ESTRIDE),
        ("s_sb", -1, ESTRIDE),
        ("o", 0x100008, EALIGN),
        ("w_v", 0x300004, EALIGN),
        ("gate", 0x500002, EALIGN),
        ("core", 0x600004, EALIGN),
        ("core", 0x600008, EALIGN),  # 16-byte output stores
        ("gate", 0x500008, EALIGN),
        ("lse", 0x200002, EALIGN),
        ("o_sj", 1 << 61, ERANGE),
        ("l_sj", 1 << 62, ERANGE),
        ("s_sv", 1 << 62, ERANGE),
    ],
)
def test_invalid_args_rejected(lib, field, value, status):
    a = good_args()
    setattr(a, field, value)
    assert check(lib, a) == status
    # mla_post validates first and returns the same status without launching
    assert lib.mla_post(ctypes.byref(a), None) == status


@pytest.mark.parametrize(
    "fields,status",
    [
        ({"q": -1}, EINVAL),
        ({"q": 3}, EINVAL),  # S = 8 is not a multiple of 3
        ({"q": 4, "o_sr": 4}, ESTRIDE),
        ({"q": 4, "o_sr": -8}, ESTRIDE),
        ({"q": 4, "l_sr": -1}, ESTRIDE),
        ({"q": 2, "kv_lens": 0x800002}, EALIGN),
        ({"qsl": 0x900001}, EALIGN),
        ({"kv_lens": 0x800000, "kl_sj": -1}, ESTRIDE),
        ({"q": 2, "o_sr": 1 << 61}, ERANGE),
        ({"q": 2, "l_sr": 1 << 61}, ERANGE),
        ({"kv_lens": 0x800000, "kl_sj": 1 << 62}, ERANGE),
    ],
)
def test_request_major_args_rejected(lib, fields, status):
    a = good_args()
    for k, v in fields.items():
        setattr(a, k, v)
    assert check(lib, a) == status


def test_request_major_args_accepted(lib):
    a = good_args(n=4, S=8)
    a.q, a.o_sr, a.l_sr = 4, 4 * 8 * 6144, 4 * 8 * 12
    a.kv_lens, a.kl_sj, a.qsl = 0x800000, 2, 0x900000
    assert check(lib, a) == OK
    a.q = 0  # 0 means one token per request
    assert check(lib, a) == OK


def test_version1_struct_ignores_later_fields(lib):
    """A version-1 caller (struct_size 176): fields past the prefix are not
    read, so junk there passes; the same junk in a full-size struct fails."""
    a = good_args()
    a.q, a.o_sr, a.kv_lens = 7, 3, 0x11
    a.struct_size = m.ARGS_V1_SIZE
    assert check(lib, a) == OK
    a.struct_size = ctypes.sizeof(m.MlaPostArgs)
    assert check(lib, a) != OK
    a.struct_size = m.ARGS_V1_SIZE - 8
    assert check(lib, a) == EINVAL


def test_debug_pointer_alignment(lib):
    a = good_args()
    a.dbg_lat = 0x700008
    assert check(lib, a) == EALIGN
    a = good_args()
    a.dbg_codes = 0x700002
    assert check(lib, a) == EALIGN
    a = good_args()
    a.dbg_lat, a.dbg_codes, a.dbg_scales = 0x700000, 0x800000, 0x900001
    assert check(lib, a) == OK


def test_null_args_pointer(lib):
    assert lib.mla_post_check(None) == EINVAL
    assert lib.mla_post(None, None) == EINVAL


def test_quantizer_validation(lib):
    q = lib.mla_quantize_mxfp4
    assert q(0x1000, 4, 500, 512, 0x2000, 256, 0x3000, 16, None) == EUNSUP  # not a multiple of 32
    assert q(0x1000, 4, 8224, 8224, 0x2000, 4112, 0x3000, 257, None) == EUNSUP  # wider than 8192
    assert q(0x1008, 4, 512, 512, 0x2000, 256, 0x3000, 16, None) == EALIGN
    assert q(0x1000, 4, 512, 500, 0x2000, 256, 0x3000, 16, None) == ESTRIDE
    assert q(0x1000, 4, 512, 512, 0x2000, 254, 0x3000, 16, None) == ESTRIDE
    assert q(None, 4, 512, 512, 0x2000, 256, 0x3000, 16, None) == EINVAL
    assert q(0x1000, -1, 512, 512, 0x2000, 256, 0x3000, 16, None) == EINVAL
    assert q(0x1000, 0, 512, 512, 0x2000, 256, 0x3000, 16, None) == OK  # nothing to do
    assert q(0x1000, 1 << 60, 512, 512, 0x2000, 256, 0x3000, 16, None) == ERANGE
    assert q(0x1000, 4, 512, 1 << 62, 0x2000, 256, 0x3000, 16, None) == ERANGE
    assert q(0x1000, (1 << 34) + 1, 512, 0, 0x2000, 0, 0x3000, 0, None) == ERANGE  # rows beyond the limit
    assert q(0x1000, (1 << 63) - 1, 512, 0, 0x2000, 0, 0x3000, 0, None) == ERANGE  # no overflow in the grid


def test_token_count_limit(lib):
    """S up to MLA_POST_SMAX = 2^30 is accepted, above it is rejected (the
    tile and token arithmetic stays far from overflow)."""
    a = good_args(n=2, S=1 << 30)
    assert check(lib, a) == OK
    a = good_args(n=2, S=(1 << 30) + 4)
    assert check(lib, a) == EINVAL
    src = open(os.path.join(ROOT, "include", "mla_post.h")).read()
    assert "#define MLA_POST_SMAX (1 << 30)" in src


# ---------------------------------------------------------------- the Python binding's checks


def cpu_inputs(n=2, S=3):
    o = torch.zeros((n, S, 12, 512), dtype=torch.bfloat16)
    lse = torch.zeros((n, S, 12), dtype=torch.float32)
    w_v = torch.zeros((12, 128, 256), dtype=torch.uint8)
    w_s = torch.full((12, 128, 16), 127, dtype=torch.uint8)
    gate = torch.zeros((S, 1536), dtype=torch.bfloat16)
    core = torch.zeros((S, 1536), dtype=torch.bfloat16)
    return o, lse, w_v, w_s, gate, core


def test_binding_type_checks():
    o, lse, w_v, w_s, gate, core = cpu_inputs()
    with pytest.raises(TypeError):
        m.make_args(o.float(), lse, w_v, w_s, gate, core)  # o must be bf16
    with pytest.raises(TypeError):
        m.make_args(o, lse.double(), w_v, w_s, gate, core)
    with pytest.raises(ValueError):
        m.make_args(o, None, w_v, w_s, gate, core)  # n = 2 needs lse
    with pytest.raises(ValueError):
        m.make_args(o.transpose(2, 3), lse, w_v, w_s, gate, core)
    with pytest.raises(ValueError):
        m.make_args(o, lse, w_v, w_s, gate.t().contiguous().t(), core)  # gate not contiguous
    with pytest.raises(ValueError):
        m.make_args(o, lse, w_v, w_s, gate, core[:2])
    with pytest.raises(TypeError):
        m.make_args(o, lse, w_v.to(torch.int8), w_s, gate, core)
    a = m.make_args(o, lse, w_v, w_s, gate, core)
    assert (a.n, a.S, a.o_sj, a.o_st, a.o_sh) == (2, 3, 3 * 6144, 6144, 512)
    assert (a.l_sj, a.l_st, a.l_sh) == (36, 12, 1)


def test_binding_refuses_cpu_tensors():
    o, lse, w_v, w_s, gate, core = cpu_inputs()
    with pytest.raises(ValueError):
        m.mla_post(o, lse, w_v, w_s, gate, core)


def test_ranks_view_strides():
    S, R = 5, 8
    buf = torch.zeros((S, 104, 512), dtype=torch.bfloat16)
    lse = torch.zeros((S, 96), dtype=torch.float32)
    ov, lv = m.ranks_view(buf, lse, R)
    assert ov.shape == (R, S, 12, 512) and ov.stride() == (12 * 512, 104 * 512, 512, 1)
    assert lv.shape == (R, S, 12) and lv.stride() == (12, 96, 1)
    buf.view(torch.int16)[3, 2 * 12 + 5, 7] = 1234
    assert ov.view(torch.int16)[2, 3, 5, 7] == 1234


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(m, "_lib", None)
    monkeypatch.setattr(m, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(FileNotFoundError):
        m.load()
