"""mla_split_kv_amd: MLA decode post-attention (LSE merge -> bf16 latents ->
MXFP4 -> FP4-MFMA W_UV -> gate) on AMD MI355X.

A thin ctypes binding over the C-ABI library ``libmla_post.so`` (declared in
``include/mla_post.h``): it checks torch tensors' dtypes, shapes and devices,
marshals pointers and strides, and enqueues the call on torch's current HIP
stream. Every step of the computation runs in the library's HIP kernels; there
is no fallback. When the library has not been built, ``load()`` raises.

The operation follows the vLLM API-docs page for module
``vllm.models.kimi_k3.amd.specialized_decode.mono.attention.mla_back``
(functions mla_post and host_args for the interface).
"""

from __future__ import annotations

import ctypes
import os

import torch  # loads torch's HIP runtime before the library resolves its own

NH, KVL, VD, GROWS = 12, 512, 128, 1536
NMAX = 512
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla_post.so")

STATUS = {
    0: "MLA_POST_OK",
    -1: "MLA_POST_EINVAL",
    -2: "MLA_POST_ESTRIDE",
    -3: "MLA_POST_EALIGN",
    -4: "MLA_POST_ERANGE",
    -5: "MLA_POST_EUNSUPPORTED",
    -6: "MLA_POST_ELAUNCH",
}


class MlaPostArgs(ctypes.Structure):
    """Mirror of ``mla_post_args`` in include/mla_post.h."""

    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("n", ctypes.c_int32),
        ("S", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("o", ctypes.c_void_p),
        ("o_sj", ctypes.c_int64),
        ("o_st", ctypes.c_int64),
        ("o_sh", ctypes.c_int64),
        ("lse", ctypes.c_void_p),
        ("l_sj", ctypes.c_int64),
        ("l_st", ctypes.c_int64),
        ("l_sh", ctypes.c_int64),
        ("w_v", ctypes.c_void_p),
        ("w_sh", ctypes.c_int64),
        ("w_sv", ctypes.c_int64),
        ("w_v_scale", ctypes.c_void_p),
        ("s_sh", ctypes.c_int64),
        ("s_sv", ctypes.c_int64),
        ("s_sb", ctypes.c_int64),
        ("gate", ctypes.c_void_p),
        ("core", ctypes.c_void_p),
        ("dbg_lat", ctypes.c_void_p),
        ("dbg_codes", ctypes.c_void_p),
        ("dbg_scales", ctypes.c_void_p),
        ("q", ctypes.c_int32),
        ("reserved2", ctypes.c_int32),
        ("o_sr", ctypes.c_int64),
        ("l_sr", ctypes.c_int64),
        ("kv_lens", ctypes.c_void_p),
        ("kl_sj", ctypes.c_int64),
        ("qsl", ctypes.c_void_p),
    ]


ARGS_V1_SIZE = 176  # MLA_POST_ARGS_V1_SIZE: the struct up to dbg_scales


class MlaDecodeArgs(ctypes.Structure):
    """Mirror of ``mla_decode_args`` in include/mla_decode.h."""

    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("R", ctypes.c_int32),
        ("q", ctypes.c_int32),
        ("n", ctypes.c_int32),
        ("qry", ctypes.c_void_p),
        ("q_st", ctypes.c_int64),
        ("q_sh", ctypes.c_int64),
        ("kv", ctypes.c_void_p),
        ("kv_st", ctypes.c_int64),
        ("indptr", ctypes.c_void_p),
        ("scale", ctypes.c_float),
        ("reserved", ctypes.c_int32),
        ("w_v", ctypes.c_void_p),
        ("w_sh", ctypes.c_int64),
        ("w_sv", ctypes.c_int64),
        ("w_v_scale", ctypes.c_void_p),
        ("s_sh", ctypes.c_int64),
        ("s_sv", ctypes.c_int64),
        ("s_sb", ctypes.c_int64),
        ("gate", ctypes.c_void_p),
        ("core", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_int64),
        ("dbg_lat", ctypes.c_void_p),
        ("dbg_codes", ctypes.c_void_p),
        ("dbg_scales", ctypes.c_void_p),
    ]


DQK = 576  # MLA_DECODE_DQK


class MlaPostPlan(ctypes.Structure):
    """mla_post_plan: the launch mla_post makes for a call."""

    _fields_ = [
        (name, ctypes.c_int32)
        for name in (
            "kernel",
            "tile_tokens",
            "rows_held",
            "lse_chunks",
            "workgroups_per_head",
            "workgroups",
            "full_tiles",
            "short_tokens",
            "pair_rows",
            "cus",
        )
    ]


KERNELS = {0: "none", 1: "one_tile", 2: "persistent", 3: "split_rows", 4: "stream"}  # MLA_POST_KERNEL_*


EXPORTS = (
    "mla_post",
    "mla_post_check",
    "mla_post_plan_for",
    "mla_quantize_mxfp4",
    "mla_post_strerror",
    "mla_post_last_hip_error",
    "mla_post_version",
    "mla_oproj",
    "mla_oproj_check",
    "mla_oproj_plan",
    "mla_decode",
    "mla_decode_partials",
    "mla_decode_check",
    "mla_decode_workspace",
    "mla_decode_workspace_init",
    "mla_decode_noalloc",
    "mla_measure_read",
)

_lib = None


class MlaPostError(RuntimeError):
    """A non-zero MLA_POST_* status from the library: `status` is the code,
    the message its name and the library's detail."""

    def __init__(self, status: int, detail: str = ""):
        self.status = status
        super().__init__(f"{STATUS.get(status, status)}: {detail}")


def load() -> ctypes.CDLL:
    """Load libmla_post.so (raises FileNotFoundError when it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise FileNotFoundError(f"{LIB_PATH} is not built: run `python -m mla_split_kv_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    lib.mla_post.argtypes = [ctypes.POINTER(MlaPostArgs), ctypes.c_void_p]
    lib.mla_post.restype = ctypes.c_int
    lib.mla_post_check.argtypes = [ctypes.POINTER(MlaPostArgs)]
    lib.mla_post_check.restype = ctypes.c_int
    lib.mla_post_plan_for.argtypes = [ctypes.POINTER(MlaPostArgs), ctypes.c_int32, ctypes.POINTER(MlaPostPlan)]
    lib.mla_post_plan_for.restype = ctypes.c_int
    lib.mla_quantize_mxfp4.argtypes = [
        ctypes.c_void_p,
        ctypes.c_int64,
        ctypes.c_int32,
        ctypes.c_int64,
        ctypes.c_void_p,
        ctypes.c_int64,
        ctypes.c_void_p,
        ctypes.c_int64,
        ctypes.c_void_p,
    ]
    lib.mla_quantize_mxfp4.restype = ctypes.c_int
    lib.mla_post_strerror.argtypes = [ctypes.c_int]
    lib.mla_post_strerror.restype = ctypes.c_char_p
    lib.mla_post_last_hip_error.argtypes = []
    lib.mla_post_last_hip_error.restype = ctypes.c_char_p
    lib.mla_post_version.argtypes = []
    lib.mla_post_version.restype = ctypes.c_int
    i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    lib.mla_oproj.argtypes = [vp, i64, i32, i32, vp, i64, i32, vp, i64, vp]
    lib.mla_oproj.restype = ctypes.c_int
    lib.mla_oproj_check.argtypes = [vp, i64, i32, i32, vp, i64, i32, vp, i64]
    lib.mla_oproj_check.restype = ctypes.c_int
    lib.mla_oproj_plan.argtypes = [i32, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.mla_oproj_plan.restype = ctypes.c_int
    for f in ("mla_decode", "mla_decode_partials"):
        getattr(lib, f).argtypes = [ctypes.POINTER(MlaDecodeArgs), vp]
        getattr(lib, f).restype = ctypes.c_int
    lib.mla_decode_check.argtypes = [ctypes.POINTER(MlaDecodeArgs)]
    lib.mla_decode_check.restype = ctypes.c_int
    pi64 = ctypes.POINTER(i64)
    lib.mla_decode_workspace.argtypes = [i32, i32, i32, pi64, pi64, pi64, pi64]
    lib.mla_decode_workspace.restype = ctypes.c_int
    lib.mla_decode_workspace_init.argtypes = [vp, i32, vp]
    lib.mla_decode_workspace_init.restype = ctypes.c_int
    lib.mla_decode_noalloc.argtypes = [ctypes.POINTER(MlaDecodeArgs), vp]
    lib.mla_decode_noalloc.restype = ctypes.c_int
    lib.mla_measure_read.argtypes = [vp, i64, vp, vp]
    lib.mla_measure_read.restype = ctypes.c_int
    _lib = lib
    return lib


def _raise(lib, st: int):
    if st != 0:
        detail = lib.mla_post_strerror(st).decode()
        if st == -6:
            detail += ": " + lib.mla_post_last_hip_error().decode()
        raise MlaPostError(st, detail)


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _need(cond: bool, exc, msg: str):
    if not cond:
        raise exc(msg)


def make_args(o, lse, w_v, w_v_scale, gate, core, dbg=None, q=1, o_sr=0, l_sr=0, kv_lens=None, qsl=None) -> MlaPostArgs:
    """Validate tensors (the checks of the page's host_args) and fill the struct.

    o      bf16 [n, S, 12, 512] view, innermost stride 1 (any other strides)
    lse    float32 [n, S, 12] view, or None when n == 1 (o is then the final
           attention output)
    w_v    uint8 [12, 128, 256] MXFP4 codes, innermost stride 1
    w_v_scale uint8 [12, 128, 16] E8M0 codes, any strides
    gate, core  bf16 [S, 1536], contiguous
    dbg    optional (lat bf16 [S,12,512], codes u8 [S,12,256], scales u8 [S,12,16])
    q, o_sr, l_sr  request-major slices: token t of request t // q reads row
           o[j, t, h] + (t // q) * o_sr elements (and likewise lse with l_sr)
    kv_lens  optional int32 [n, S // q] (or [S // q], shared): 0 marks the
           partial of that request empty (the page's stage_push masking)
    qsl    optional int32 [S // q + 1]: tokens >= qsl[S // q] are past the batch
    """
    _need(o.dim() == 4 and o.shape[2:] == (NH, KVL), ValueError, f"o must be [n, S, 12, 512], got {tuple(o.shape)}")
    n, S = int(o.shape[0]), int(o.shape[1])
    _need(o.dtype == torch.bfloat16, TypeError, "o must be bfloat16")
    _need(o.stride(-1) == 1, ValueError, "o's innermost stride must be 1")
    if lse is None:
        _need(n == 1, ValueError, "lse may be omitted only with one partial")
    else:
        _need(lse.dtype == torch.float32, TypeError, "lse must be float32")
        _need(tuple(lse.shape) == (n, S, NH), ValueError, f"lse must be [{n}, {S}, 12], got {tuple(lse.shape)}")
    _need(w_v.dtype == torch.uint8 and tuple(w_v.shape) == (NH, VD, KVL // 2), TypeError, "w_v must be uint8 [12,128,256]")
    _need(w_v.stride(-1) == 1, ValueError, "w_v's innermost stride must be 1")
    _need(
        w_v_scale.dtype == torch.uint8 and tuple(w_v_scale.shape) == (NH, VD, KVL // 32),
        TypeError,
        "w_v_scale must be uint8 [12,128,16]",
    )
    for name, t in (("gate", gate), ("core", core)):
        _need(t.dtype == torch.bfloat16, TypeError, f"{name} must be bfloat16")
        _need(tuple(t.shape) == (S, GROWS), ValueError, f"{name} must be [{S}, 1536], got {tuple(t.shape)}")
        _need(t.is_contiguous(), ValueError, f"{name} must be contiguous")
    dev = core.device
    tensors = [o, w_v, w_v_scale, gate, core] + ([] if lse is None else [lse])
    _need(all(t.device == dev for t in tensors), ValueError, "all tensors must be on one device")
    a = MlaPostArgs()
    a.struct_size = ctypes.sizeof(MlaPostArgs)
    a.n, a.S = n, S
    a.o = o.data_ptr()
    a.o_sj, a.o_st, a.o_sh = o.stride(0), o.stride(1), o.stride(2)
    if lse is not None:
        a.lse = lse.data_ptr()
        a.l_sj, a.l_st, a.l_sh = lse.stride(0), lse.stride(1), lse.stride(2)
    a.w_v = w_v.data_ptr()
    a.w_sh, a.w_sv = w_v.stride(0), w_v.stride(1)
    a.w_v_scale = w_v_scale.data_ptr()
    a.s_sh, a.s_sv, a.s_sb = w_v_scale.stride(0), w_v_scale.stride(1), w_v_scale.stride(2)
    a.gate = gate.data_ptr()
    a.core = core.data_ptr()
    _need(q >= 1 and S % q == 0, ValueError, f"S={S} must be a multiple of q={q}")
    a.q, a.o_sr, a.l_sr = q, o_sr, l_sr
    R = S // q
    if kv_lens is not None:
        _need(kv_lens.dtype == torch.int32 and kv_lens.device == dev, TypeError, "kv_lens must be int32 on the device")
        if kv_lens.dim() == 1:
            _need(kv_lens.shape[0] == R and kv_lens.stride(0) == 1, ValueError, "kv_lens must be [S // q]")
            a.kl_sj = 0
        else:
            _need(tuple(kv_lens.shape) == (n, R) and kv_lens.stride(1) == 1, ValueError, f"kv_lens must be [{n}, {R}]")
            a.kl_sj = kv_lens.stride(0)
        a.kv_lens = kv_lens.data_ptr()
    if qsl is not None:
        _need(qsl.dtype == torch.int32 and qsl.device == dev, TypeError, "qsl must be int32 on the device")
        _need(tuple(qsl.shape) == (R + 1,) and qsl.is_contiguous(), ValueError, f"qsl must be [{R + 1}]")
        a.qsl = qsl.data_ptr()
    if dbg is not None:
        lat, codes, scales = dbg
        _need(lat.dtype == torch.bfloat16 and tuple(lat.shape) == (S, NH, KVL) and lat.is_contiguous(), ValueError, "dbg lat")
        _need(codes.dtype == torch.uint8 and tuple(codes.shape) == (S, NH, KVL // 2) and codes.is_contiguous(), ValueError, "dbg codes")
        _need(scales.dtype == torch.uint8 and tuple(scales.shape) == (S, NH, KVL // 32) and scales.is_contiguous(), ValueError, "dbg scales")
        a.dbg_lat, a.dbg_codes, a.dbg_scales = lat.data_ptr(), codes.data_ptr(), scales.data_ptr()
    return a


def plan_args(a: MlaPostArgs, cus: int = 0) -> dict:
    """mla_post_plan_for on a filled struct: the launch mla_post would make on
    a device with ``cus`` compute units (0: the current device). Host only."""
    lib = load()
    out = MlaPostPlan()
    _raise(lib, lib.mla_post_plan_for(ctypes.byref(a), int(cus), ctypes.byref(out)))
    d = {name: getattr(out, name) for name, _ in MlaPostPlan._fields_}
    d["kernel"] = KERNELS[d["kernel"]]
    return d


def plan(o, lse, w_v, w_v_scale, gate, core=None, cus: int = 0, **layout) -> dict:
    """The launch mla_post would make for these tensors (same arguments as
    mla_post; nothing is launched and no device memory is touched)."""
    return plan_args(make_args(o, lse, w_v, w_v_scale, gate, gate if core is None else core, **layout), cus)


def mla_post(o, lse, w_v, w_v_scale, gate, core=None, debug: bool = False, **layout):
    """One mla_post call on torch's current stream of core's device.

    Returns core (bf16 [S, 1536]); with ``debug=True`` returns
    (core, latents bf16 [S,12,512], codes u8 [S,12,256], scales u8 [S,12,16]),
    all written by the same kernel launch. ``layout`` takes the request-major
    and masking arguments of make_args (q, o_sr, l_sr, kv_lens, qsl).
    """
    lib = load()
    S = int(o.shape[1])
    if core is None:
        core = torch.empty((S, GROWS), dtype=torch.bfloat16, device=gate.device)
    dbg = None
    if debug:
        dev = core.device
        dbg = (
            torch.empty((S, NH, KVL), dtype=torch.bfloat16, device=dev),
            torch.empty((S, NH, KVL // 2), dtype=torch.uint8, device=dev),
            torch.empty((S, NH, KVL // 32), dtype=torch.uint8, device=dev),
        )
    a = make_args(o, lse, w_v, w_v_scale, gate, core, dbg, **layout)
    _need(core.is_cuda, ValueError, "tensors must be on a GPU")
    _raise(lib, lib.mla_post(ctypes.byref(a), ctypes.c_void_p(_stream(core.device))))
    return core if not debug else (core,) + dbg


class Prepared:
    """A validated mla_post call whose argument struct is built once; calling
    it enqueues the kernel on torch's current stream (for timing loops and
    serving loops that reuse the same buffers)."""

    def __init__(self, o, lse, w_v, w_v_scale, gate, core, dbg=None, **layout):
        self._lib = load()
        _need(core.is_cuda, ValueError, "tensors must be on a GPU")
        self._keep = (o, lse, w_v, w_v_scale, gate, core, dbg, layout)
        self.args = make_args(o, lse, w_v, w_v_scale, gate, core, dbg, **layout)
        self._ref = ctypes.byref(self.args)
        self.device = core.device
        _raise(self._lib, self._lib.mla_post_check(self._ref))

    def __call__(self, stream: int | None = None):
        s = _stream(self.device) if stream is None else stream
        st = self._lib.mla_post(self._ref, ctypes.c_void_p(s))
        if st:
            _raise(self._lib, st)


def prepare(o, lse, w_v, w_v_scale, gate, core, **layout):
    """A validated mla_post call on these tensors, to be launched again and
    again (`Prepared`): the arguments are checked and marshalled once."""
    return Prepared(o, lse, w_v, w_v_scale, gate, core, **layout)


def mla_post_splits(o, lse, w_v, w_v_scale, gate, core=None, debug=False):
    """Split-KV partials: o [P, S, 12, 512], lse [P, S, 12] (token t merges o[:, t])."""
    return mla_post(o, lse, w_v, w_v_scale, gate, core, debug)


def request_major_layout(o_all, lse_all, q: int):
    """The page's dense split layout: o_all [P, S, 12, 512], lse_all [P, S, 12]
    with per = P / (S / q) slices for each request of q tokens, request-major;
    token t merges slices (t // q) * per + j. Returns (o view [per, S, 12, 512],
    lse view [per, S, 12], layout kwargs for mla_post)."""
    P, S = int(o_all.shape[0]), int(o_all.shape[1])
    _need(q >= 1 and S % q == 0 and P % (S // q) == 0, ValueError, "P and S must split evenly into S // q requests")
    per = P // (S // q)
    so, sl = o_all.stride(), lse_all.stride()
    ov = o_all.as_strided((per, S, NH, KVL), so, o_all.storage_offset())
    lv = lse_all.as_strided((per, S, NH), sl, lse_all.storage_offset())
    return ov, lv, {"q": q, "o_sr": per * so[0], "l_sr": per * sl[0]}


def mla_post_request_major(o_all, lse_all, q: int, w_v, w_v_scale, gate, core=None, debug=False, kv_lens=None, qsl=None):
    """Split partials in the page's request-major layout (see request_major_layout)."""
    ov, lv, lay = request_major_layout(o_all, lse_all, q)
    return mla_post(ov, lv, w_v, w_v_scale, gate, core, debug, kv_lens=kv_lens, qsl=qsl, **lay)


def ranks_view(o_gathered, lse_gathered, ranks: int):
    """Views [R, S, 12, 512] / [R, S, 12] of decode-context-parallel partials
    gathered as o [S, >= R*12, 512] and lse [S, >= R*12]: rank r's partial of
    local head h is gathered head r*12 + h (the page's mla_post layout)."""
    S = o_gathered.shape[0]
    _need(o_gathered.shape[1] >= ranks * NH and o_gathered.shape[2] == KVL, ValueError, "o must be [S, >= R*12, 512]")
    so = o_gathered.stride()
    ov = o_gathered.as_strided((ranks, S, NH, KVL), (NH * so[1], so[0], so[1], so[2]), o_gathered.storage_offset())
    lv = None
    if lse_gathered is not None:
        sl = lse_gathered.stride()
        lv = lse_gathered.as_strided((ranks, S, NH), (NH * sl[1], sl[0], sl[1]), lse_gathered.storage_offset())
    return ov, lv


def mla_post_ranks(o_gathered, lse_gathered, ranks: int, w_v, w_v_scale, gate, core=None, debug=False):
    """Decode-context-parallel merge of R gathered rank partials, in rank order."""
    ov, lv = ranks_view(o_gathered, lse_gathered, ranks)
    return mla_post(ov, lv, w_v, w_v_scale, gate, core, debug)


def quantize_mxfp4(x):
    """bf16 [rows, cols] (cols % 32 == 0, innermost stride 1) -> (codes uint8
    [rows, cols/2], scales uint8 [rows, cols/32]) with the kernel's own rule."""
    lib = load()
    _need(x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1, TypeError, "x must be bf16 [rows, cols]")
    rows, cols = int(x.shape[0]), int(x.shape[1])
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=x.device)
    st = lib.mla_quantize_mxfp4(
        ctypes.c_void_p(x.data_ptr()),
        rows,
        cols,
        x.stride(0),
        ctypes.c_void_p(codes.data_ptr()),
        codes.stride(0),
        ctypes.c_void_p(scales.data_ptr()),
        scales.stride(0),
        ctypes.c_void_p(_stream(x.device)),
    )
    _raise(lib, st)
    return codes, scales


# ---------------------------------------------------------------- o_proj (include/mla_oproj.h)


def _oproj_args(core, w_o, out):
    _need(core.dtype == torch.bfloat16 and core.dim() == 2 and core.stride(1) == 1, TypeError,
          "core must be bf16 [S, K] with unit innermost stride")
    _need(w_o.dtype == torch.bfloat16 and w_o.dim() == 2 and w_o.stride(1) == 1, TypeError,
          "w_o must be bf16 [D, K] with unit innermost stride")
    S, K = int(core.shape[0]), int(core.shape[1])
    D = int(w_o.shape[0])
    _need(int(w_o.shape[1]) == K, ValueError, f"w_o must be [D, {K}], got {tuple(w_o.shape)}")
    _need(out.dtype == torch.bfloat16 and tuple(out.shape) == (S, D) and out.stride(1) == 1, ValueError,
          f"out must be bf16 [{S}, {D}] with unit innermost stride")
    _need(core.device == w_o.device == out.device, ValueError, "all tensors must be on one device")
    return (ctypes.c_void_p(core.data_ptr()), core.stride(0), S, K, ctypes.c_void_p(w_o.data_ptr()), w_o.stride(0), D,
            ctypes.c_void_p(out.data_ptr()), out.stride(0))


def oproj(core, w_o, out=None):
    """o_proj on torch's current stream: out [S, D] = bf16(core [S, K] @ w_o[D, K]^T)
    (include/mla_oproj.h); returns out."""
    lib = load()
    if out is None:
        out = torch.empty((int(core.shape[0]), int(w_o.shape[0])), dtype=torch.bfloat16, device=core.device)
    args = _oproj_args(core, w_o, out)
    _need(core.is_cuda, ValueError, "tensors must be on a GPU")
    _raise(lib, lib.mla_oproj(*args, ctypes.c_void_p(_stream(core.device))))
    return out


def oproj_plan(S: int, D: int, cus: int = 0) -> dict:
    """The tile and grid mla_oproj uses for S x D (host only)."""
    lib = load()
    tm, tn, wg = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _raise(lib, lib.mla_oproj_plan(int(S), int(D), int(cus), ctypes.byref(tm), ctypes.byref(tn), ctypes.byref(wg)))
    return {"tile_m": tm.value, "tile_n": tn.value, "workgroups": wg.value}


class PreparedOproj:
    """A validated o_proj call whose arguments are marshalled once."""

    def __init__(self, core, w_o, out):
        self._lib = load()
        _need(core.is_cuda, ValueError, "tensors must be on a GPU")
        self._keep = (core, w_o, out)
        self.args = _oproj_args(core, w_o, out)
        self.device = core.device
        _raise(self._lib, self._lib.mla_oproj_check(*self.args))

    def __call__(self, stream: int | None = None):
        s = _stream(self.device) if stream is None else stream
        st = self._lib.mla_oproj(*self.args, ctypes.c_void_p(s))
        if st:
            _raise(self._lib, st)


# ---------------------------------------------------------------- split-KV attention fused with mla_post (include/mla_decode.h)


def decode_workspace_layout(R: int, q: int, n: int) -> dict:
    """Bytes and part offsets of mla_decode's workspace (host only)."""
    lib = load()
    b, c, p, l = (ctypes.c_int64() for _ in range(4))
    _raise(lib, lib.mla_decode_workspace(int(R), int(q), int(n), ctypes.byref(b), ctypes.byref(c), ctypes.byref(p), ctypes.byref(l)))
    return {"bytes": b.value, "counters": c.value, "partials": p.value, "lse": l.value}


class DecodeWorkspace:
    """A device workspace for mla_decode calls of R requests, q tokens, n
    splits: a uint8 tensor of the library's size (allocated by torch, not by
    the library), its counters zeroed once by mla_decode_workspace_init."""

    def __init__(self, R: int, q: int, n: int, device="cuda"):
        lib = load()
        self.R, self.q, self.n = int(R), int(q), int(n)
        self.layout = decode_workspace_layout(R, q, n)
        self.buf = torch.empty(self.layout["bytes"] + 256, dtype=torch.uint8, device=device)
        off = (-self.buf.data_ptr()) % 256
        self.mem = self.buf[off : off + self.layout["bytes"]]
        _raise(lib, lib.mla_decode_workspace_init(ctypes.c_void_p(self.mem.data_ptr()), self.R, ctypes.c_void_p(_stream(self.mem.device))))

    def counters(self):
        """int32 [R + 2]: the request counters, then the unit queue's two."""
        c = self.layout["counters"]
        return self.mem[c : c + 4 * (self.R + 2)].view(torch.int32)

    def partials(self):
        """(o bf16 [R, n, q, 12, 512], lse float32 [R, n, q, 12]) views."""
        p, l = self.layout["partials"], self.layout["lse"]
        rows = self.R * self.n * self.q * NH
        o = self.mem[p : p + rows * KVL * 2].view(torch.bfloat16).view(self.R, self.n, self.q, NH, KVL)
        lse = self.mem[l : l + rows * 4].view(torch.float32).view(self.R, self.n, self.q, NH)
        return o, lse

    def token_views(self):
        """The partials as mla_post takes them: o [n, S, 12, 512] and lse
        [n, S, 12] strided views plus the request-major layout arguments."""
        o, lse = self.partials()
        S = self.R * self.q
        so, sl = o.stride(), lse.stride()
        ov = o.as_strided((self.n, S, NH, KVL), (so[1], so[2], so[3], 1), o.storage_offset())
        lv = lse.as_strided((self.n, S, NH), (sl[1], sl[2], sl[3]), lse.storage_offset())
        lay = {"q": self.q, "o_sr": so[0] - self.q * so[2], "l_sr": sl[0] - self.q * sl[2]}
        return ov, lv, lay


def _decode_args(qry, kv, indptr, q, n, scale, w_v, w_v_scale, gate, core, ws, dbg=None) -> MlaDecodeArgs:
    _need(qry.dtype == torch.bfloat16 and qry.dim() == 3 and tuple(qry.shape[1:]) == (NH, DQK) and qry.stride(2) == 1,
          TypeError, "qry must be bf16 [S, 12, 576] with unit innermost stride")
    _need(kv.dtype == torch.bfloat16 and kv.dim() == 2 and kv.shape[1] == DQK and kv.stride(1) == 1, TypeError,
          "kv must be bf16 [rows, 576] with unit innermost stride")
    _need(indptr.dtype == torch.int32 and indptr.dim() == 1 and indptr.is_contiguous(), TypeError, "indptr must be int32 [R + 1]")
    R = int(indptr.shape[0]) - 1
    S = int(qry.shape[0])
    _need(R >= 0 and S == R * q, ValueError, f"qry has {S} tokens, expected R * q = {R * q}")
    _need((ws.R, ws.q, ws.n) == (R, q, n), ValueError, "workspace made for another (R, q, n)")
    _need(w_v.dtype == torch.uint8 and tuple(w_v.shape) == (NH, VD, KVL // 2) and w_v.stride(-1) == 1, TypeError,
          "w_v must be uint8 [12,128,256]")
    _need(w_v_scale.dtype == torch.uint8 and tuple(w_v_scale.shape) == (NH, VD, KVL // 32), TypeError,
          "w_v_scale must be uint8 [12,128,16]")
    for name, t in (("gate", gate), ("core", core)):
        _need(t.dtype == torch.bfloat16 and tuple(t.shape) == (S, GROWS) and t.is_contiguous(), ValueError,
              f"{name} must be contiguous bf16 [{S}, 1536]")
    a = MlaDecodeArgs()
    a.struct_size = ctypes.sizeof(MlaDecodeArgs)
    a.R, a.q, a.n = R, int(q), int(n)
    a.qry, a.q_st, a.q_sh = qry.data_ptr(), qry.stride(0), qry.stride(1)
    a.kv, a.kv_st = kv.data_ptr(), kv.stride(0)
    a.indptr = indptr.data_ptr()
    a.scale = float(scale)
    a.w_v, a.w_sh, a.w_sv = w_v.data_ptr(), w_v.stride(0), w_v.stride(1)
    a.w_v_scale = w_v_scale.data_ptr()
    a.s_sh, a.s_sv, a.s_sb = w_v_scale.stride(0), w_v_scale.stride(1), w_v_scale.stride(2)
    a.gate, a.core = gate.data_ptr(), core.data_ptr()
    a.workspace, a.workspace_bytes = ws.mem.data_ptr(), ws.layout["bytes"]
    if dbg is not None:
        a.dbg_lat, a.dbg_codes, a.dbg_scales = (t.data_ptr() for t in dbg)
    return a


def mla_decode(qry, kv, indptr, q: int, n: int, scale: float, w_v, w_v_scale, gate, ws: DecodeWorkspace, core=None,
               debug: bool = False, fused: bool = True):
    """Split-KV MLA decode attention and mla_post on torch's current stream.

    fused=True: one launch (include/mla_decode.h's mla_decode); returns core
    (with debug=True: core, latents, codes, scales of the merge).
    fused=False: the attention alone (mla_decode_partials); its partials are
    left in ws (ws.partials(), ws.token_views()) and core is not written."""
    lib = load()
    S = int(qry.shape[0])
    if core is None:
        core = torch.empty((S, GROWS), dtype=torch.bfloat16, device=gate.device)
    dbg = None
    if debug:
        dev = core.device
        dbg = (torch.empty((S, NH, KVL), dtype=torch.bfloat16, device=dev),
               torch.empty((S, NH, KVL // 2), dtype=torch.uint8, device=dev),
               torch.empty((S, NH, KVL // 32), dtype=torch.uint8, device=dev))
    a = _decode_args(qry, kv, indptr, q, n, scale, w_v, w_v_scale, gate, core, ws, dbg)
    _need(core.is_cuda, ValueError, "tensors must be on a GPU")
    f = lib.mla_decode if fused else lib.mla_decode_partials
    _raise(lib, f(ctypes.byref(a), ctypes.c_void_p(_stream(core.device))))
    return core if not debug else (core,) + dbg


DECODE_SCRATCH_BYTES = 64 << 20  # MLA_DECODE_SCRATCH_BYTES


class _NoWorkspace:
    """Stands in for a DecodeWorkspace in mla_decode_noalloc's arguments."""

    def __init__(self, R, q, n):
        self.R, self.q, self.n = R, q, n
        self.layout = {"bytes": 0}
        self.mem = type("_Null", (), {"data_ptr": staticmethod(lambda: 0)})()


def mla_decode_noalloc(qry, kv, indptr, q: int, n: int, scale: float, w_v, w_v_scale, gate, core=None):
    """The fused launch with the library's own scratch array as workspace
    (include/mla_decode.h's mla_decode_noalloc): nothing is allocated by the
    library; returns core (allocated here by torch when not given)."""
    lib = load()
    S = int(qry.shape[0])
    if core is None:
        core = torch.empty((S, GROWS), dtype=torch.bfloat16, device=gate.device)
    R = int(indptr.shape[0]) - 1
    a = _decode_args(qry, kv, indptr, q, n, scale, w_v, w_v_scale, gate, core, _NoWorkspace(R, q, n))
    _need(core.is_cuda, ValueError, "tensors must be on a GPU")
    _raise(lib, lib.mla_decode_noalloc(ctypes.byref(a), ctypes.c_void_p(_stream(core.device))))
    return core


class PreparedDecode:
    """A validated mla_decode call (fused or the attention alone) whose
    argument struct is built once."""

    def __init__(self, qry, kv, indptr, q, n, scale, w_v, w_v_scale, gate, ws, core, fused=True):
        self._lib = load()
        self._keep = (qry, kv, indptr, w_v, w_v_scale, gate, ws, core)
        self.args = _decode_args(qry, kv, indptr, q, n, scale, w_v, w_v_scale, gate, core, ws)
        self._ref = ctypes.byref(self.args)
        self.device = core.device
        self._f = self._lib.mla_decode if fused else self._lib.mla_decode_partials
        _raise(self._lib, self._lib.mla_decode_check(self._ref))

    def __call__(self, stream: int | None = None):
        s = _stream(self.device) if stream is None else stream
        st = self._f(self._ref, ctypes.c_void_p(s))
        if st:
            _raise(self._lib, st)


# ---------------------------------------------------------------- bandwidth reference (include/mla_measure.h)


def measure_read(t, sink=None):
    """Read tensor t's bytes once (include/mla_measure.h's mla_measure_read) on
    torch's current stream: the plain-read reference of the benchmark."""
    lib = load()
    _need(t.is_cuda and t.is_contiguous(), ValueError, "t must be a contiguous GPU tensor")
    if sink is None:
        sink = torch.empty(16, dtype=torch.uint8, device=t.device)
    n = t.numel() * t.element_size()
    _raise(lib, lib.mla_measure_read(ctypes.c_void_p(t.data_ptr()), n, ctypes.c_void_p(sink.data_ptr()),
                                     ctypes.c_void_p(_stream(t.device))))
