"""Python binding of libmxattn.so (MXFP4 FlashAttention for MI355X / gfx950).

Argument marshalling only: every step runs in the HIP library.  torch tensors
provide device memory and the current stream.  If the shared library is
missing the import fails; there is no fallback path.

    import bit_microscaled_flashattention_amd as mxa
    qh = mxa.quantize(q)                        # [B,H,S,D] bf16 -> MXFP4 (HD)
    vh = mxa.quantize(v, layout="key")          # 32-key blocks per channel
    out = mxa.prefill(qh, kh, vh, causal=True)
"""

import ctypes
import math
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MXATTN_LIBRARY selects another build of the library (same ABI).
LIB_PATH = os.environ.get("MXATTN_LIBRARY") or os.path.join(_HERE, "libmxattn.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(5)
F32, F16, BF16 = 0, 1, 2
SCALE_OCP, SCALE_UOS = 0, 1
LAYOUT_HD, LAYOUT_KEY = 0, 1
UOS_QMAX = 7.25

_DT = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
_RULES = {"ocp": SCALE_OCP, "uos": SCALE_UOS}


class MxattnError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"mxattn status {status}: {message}")
        self.status = status


class _Mx(ctypes.Structure):
    _fields_ = [
        ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
        ("batch", ctypes.c_int64), ("heads", ctypes.c_int64),
        ("seq", ctypes.c_int64), ("dim", ctypes.c_int64),
        ("layout", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("code_stride", ctypes.c_int64 * 3), ("scale_stride", ctypes.c_int64 * 3),
    ]


class _QuantJob(ctypes.Structure):
    _fields_ = [
        ("x", ctypes.c_void_p), ("x_dtype", ctypes.c_int32), ("flags", ctypes.c_int32),
        ("x_stride", ctypes.c_int64 * 3), ("chan_scale", ctypes.c_void_p),
        ("rule", ctypes.c_int32), ("qmax", ctypes.c_float), ("out", ctypes.POINTER(_Mx)),
    ]


MAX_QUANTIZE_JOBS = 4


class _PrefillParams(ctypes.Structure):
    _fields_ = [
        ("causal", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
        ("kv_tile", ctypes.c_int32), ("p_rule", ctypes.c_int32),
        ("p_qmax", ctypes.c_float), ("l_from_quantized", ctypes.c_int32),
    ]


class _PrefillHybrid(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("idx", ctypes.c_void_p), ("n_sel", ctypes.c_void_p),
        ("max_sel", ctypes.c_int32), ("window", ctypes.c_int32),
    ]


class _Paging(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("max_pages", ctypes.c_int32)]


class _Hybrid(ctypes.Structure):
    _fields_ = [
        ("idx", ctypes.c_void_p), ("n_sel", ctypes.c_void_p),
        ("max_sel", ctypes.c_int32), ("window", ctypes.c_int32),
        ("k_sel", ctypes.c_void_p), ("v_sel", ctypes.c_void_p),
        ("k_win", ctypes.c_void_p), ("v_win", ctypes.c_void_p),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run python -m bit_microscaled_flashattention_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    P = ctypes.POINTER
    sig = {
        "mxattn_quantize": [vp, i32, P(i64), vp, i32, f32, i32, P(_Mx), vp],
        "mxattn_quantize_batch": [P(_QuantJob), i32, vp],
        "mxattn_smooth_calibrate": [vp, vp, i32, i64, i64, i64, i64, vp, vp, vp],
        "mxattn_prefill": [P(_Mx), P(_Mx), P(_Mx), P(_PrefillParams), vp, i32, vp, vp],
        "mxattn_prefill_hybrid": [P(_Mx), P(_Mx), P(_Mx), P(_PrefillParams), P(_PrefillHybrid), vp, i32, vp, vp],
        "mxattn_decode": [P(_Mx), P(_Mx), vp, P(_Mx), P(_Mx), vp, P(_Hybrid), f32, i32, vp, sz, vp, vp, vp],
        "mxattn_decode_paged": [P(_Mx), P(_Mx), vp, P(_Mx), P(_Mx), P(_Paging), vp, P(_Hybrid), f32, i32, vp, sz,
                                vp, vp, vp],
        "mxattn_decode_noalloc": [P(_Mx), P(_Mx), vp, P(_Mx), P(_Mx), vp, P(_Hybrid), f32, i32, vp, vp, vp],
        "mxattn_gather_rows": [vp, vp, P(i64), P(i64), P(i64), vp, vp, i32, vp, vp, vp],
        "mxattn_quantize_dual": [vp, i32, P(i64), vp, i32, f32, i32, P(_Mx), P(_Mx), vp],
        "mxattn_select_vertical": [P(_Mx), P(_Mx), vp, f32, i32, i32, i32, vp, vp, vp, i32, vp, sz, vp],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = i32
    lib.mxattn_decode_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i32, i32]
    lib.mxattn_decode_workspace_bytes.restype = sz
    lib.mxattn_select_workspace_bytes.argtypes = [i64, i64, i64, i64]
    lib.mxattn_select_workspace_bytes.restype = sz
    for name in ("mxattn_last_error", "mxattn_version"):
        getattr(lib, name).restype = ctypes.c_char_p
        getattr(lib, name).argtypes = []
    lib.mxattn_status_string.restype = ctypes.c_char_p
    lib.mxattn_status_string.argtypes = [i32]
    return lib


_lib = _load()

# Every symbol the C header declares (checked by the CPU tests).
EXPORTS = (
    "mxattn_quantize", "mxattn_quantize_dual", "mxattn_quantize_batch", "mxattn_smooth_calibrate", "mxattn_prefill",
    "mxattn_prefill_hybrid",
    "mxattn_decode_workspace_bytes", "mxattn_decode", "mxattn_decode_paged", "mxattn_decode_noalloc",
    "mxattn_select_workspace_bytes", "mxattn_select_vertical", "mxattn_gather_rows",
    "mxattn_status_string", "mxattn_last_error", "mxattn_version",
)


def library():
    return _lib


def version():
    return _lib.mxattn_version().decode()


def _check(status):
    if status != OK:
        raise MxattnError(status, _lib.mxattn_last_error().decode())


def _stream(t=None):
    if t is not None and t.is_cuda:
        return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)
    return ctypes.c_void_p(0)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


@dataclass
class MX:
    """An MXFP4 tensor: packed E2M1 codes + E8M0 scale bytes (torch uint8).

    layout "hd":  codes [B,H,S,D/2], scales [B,H,S,D/32]
    layout "key": codes [B,H,D,ceil(S/32)*16], scales [B,H,D,ceil(S/32)]
    """
    codes: torch.Tensor
    scales: torch.Tensor
    shape: tuple
    layout: str = "hd"

    def desc(self):
        """C descriptor; an MX without codes (None) describes only a shape."""
        b, h, s, d = self.shape
        c, sc = self.codes, self.scales
        m = _Mx()
        m.batch, m.heads, m.seq, m.dim = b, h, s, d
        m.layout = LAYOUT_HD if self.layout == "hd" else LAYOUT_KEY
        if c is None:
            return m
        m.codes, m.scales = c.data_ptr(), sc.data_ptr()
        for i in range(3):
            m.code_stride[i] = c.stride(i) * c.element_size()
            m.scale_stride[i] = sc.stride(i) * sc.element_size()
        return m

    def narrow_seq(self, start, length):
        """View of tokens [start, start+length) of an HD tensor (no copy)."""
        assert self.layout == "hd"
        b, h, _, d = self.shape
        return MX(self.codes[:, :, start:start + length], self.scales[:, :, start:start + length],
                  (b, h, length, d), "hd")


def empty_mx(shape, layout="hd", device="cuda"):
    b, h, s, d = shape
    if layout == "hd":
        codes = torch.empty((b, h, s, d // 2), dtype=torch.uint8, device=device)
        scales = torch.empty((b, h, s, d // 32), dtype=torch.uint8, device=device)
    else:
        nb = (s + 31) // 32
        codes = torch.empty((b, h, d, nb * 16), dtype=torch.uint8, device=device)
        scales = torch.empty((b, h, d, nb), dtype=torch.uint8, device=device)
    return MX(codes, scales, tuple(shape), layout)


QUANT_HADAMARD = 1


def quantize(x, layout="hd", chan_scale=None, rule="ocp", qmax=UOS_QMAX, out=None, hadamard=False):
    """MXFP4-encode x [B,H,S,D] (bf16/fp16/fp32, last dim contiguous).
    hadamard=True rotates each head-dim row first (rotate Q and K alike)."""
    assert x.dim() == 4 and x.stride(3) == 1, "x must be [B,H,S,D] with contiguous D"
    if out is None:
        out = empty_mx(tuple(x.shape), layout, x.device)
    strides = (ctypes.c_int64 * 3)(x.stride(0), x.stride(1), x.stride(2))
    cs = None
    if chan_scale is not None:
        cs = chan_scale.to(torch.float32).contiguous()
    d = out.desc()
    _check(_lib.mxattn_quantize(_ptr(x), _DT[x.dtype], strides, _ptr(cs), _RULES[rule],
                                float(qmax), QUANT_HADAMARD if hadamard else 0, ctypes.byref(d), _stream(x)))
    return out


def quantize_dual(x, chan_scale=None, rule="ocp", qmax=UOS_QMAX, out=None, out_res=None, hadamard=False):
    """Dual-residual MXFP4 of x [B,H,S,D] (HD blocks): returns (q1, q2) with
    q1 = quantize(x) and q2 the MXFP4 of x - dequant(q1)."""
    assert x.dim() == 4 and x.stride(3) == 1, "x must be [B,H,S,D] with contiguous D"
    if out is None:
        out = empty_mx(tuple(x.shape), "hd", x.device)
    if out_res is None:
        out_res = empty_mx(tuple(x.shape), "hd", x.device)
    strides = (ctypes.c_int64 * 3)(x.stride(0), x.stride(1), x.stride(2))
    cs = chan_scale.to(torch.float32).contiguous() if chan_scale is not None else None
    d1, d2 = out.desc(), out_res.desc()
    _check(_lib.mxattn_quantize_dual(_ptr(x), _DT[x.dtype], strides, _ptr(cs), _RULES[rule], float(qmax),
                                     QUANT_HADAMARD if hadamard else 0, ctypes.byref(d1), ctypes.byref(d2),
                                     _stream(x)))
    return out, out_res


def quantize_batch(jobs):
    """Several quantize() calls in one launch.  jobs: list of dicts with the
    keyword arguments of quantize() (x required; layout, chan_scale, rule,
    qmax, out optional).  Returns the outputs in job order; bit-identical to
    one quantize() per job."""
    assert 1 <= len(jobs) <= MAX_QUANTIZE_JOBS, f"1..{MAX_QUANTIZE_JOBS} jobs"
    arr = (_QuantJob * len(jobs))()
    keep, outs = [], []
    for i, j in enumerate(jobs):
        x = j["x"]
        assert x.dim() == 4 and x.stride(3) == 1, "x must be [B,H,S,D] with contiguous D"
        out = j.get("out")
        if out is None:
            out = empty_mx(tuple(x.shape), j.get("layout", "hd"), x.device)
        cs = j.get("chan_scale")
        if cs is not None:
            cs = cs.to(torch.float32).contiguous()
        d = out.desc()
        keep += [cs, d]
        arr[i].x = _ptr(x)
        arr[i].x_dtype = _DT[x.dtype]
        arr[i].x_stride[:] = [x.stride(0), x.stride(1), x.stride(2)]
        arr[i].chan_scale = _ptr(cs)
        arr[i].rule = _RULES[j.get("rule", "ocp")]
        arr[i].qmax = float(j.get("qmax", UOS_QMAX))
        arr[i].flags = QUANT_HADAMARD if j.get("hadamard", False) else 0
        arr[i].out = ctypes.pointer(d)
        outs.append(out)
    _check(_lib.mxattn_quantize_batch(arr, len(jobs), _stream(jobs[0]["x"])))
    return outs


def smooth_calibrate(q_cal, k_cal):
    """Smooth-QK factors from calibration slices q_cal [Hq,T,D], k_cal [Hkv,T,D]."""
    q_cal, k_cal = q_cal.contiguous(), k_cal.contiguous()
    hq, t, d = q_cal.shape
    hkv = k_cal.shape[0]
    qs = torch.empty((hq, d), dtype=torch.float32, device=q_cal.device)
    ks = torch.empty((hkv, d), dtype=torch.float32, device=q_cal.device)
    _check(_lib.mxattn_smooth_calibrate(_ptr(q_cal), _ptr(k_cal), _DT[q_cal.dtype], hq, hkv, t, d,
                                        _ptr(qs), _ptr(ks), _stream(q_cal)))
    return qs, ks


def prefill(q, k, v, causal=False, softmax_scale=0.0, kv_tile=128, p_rule="ocp",
            p_qmax=UOS_QMAX, l_from_quantized=True, out_dtype=torch.float32, return_lse=False,
            out=None):
    """MXFP4 attention forward; q, k: MX (hd), v: MX (key).  Returns out [B,Hq,Sq,D]."""
    b, hq, sq, d = q.shape
    if out is None:
        out = torch.empty((b, hq, sq, d), dtype=out_dtype, device=q.codes.device)
    lse = torch.empty((b, hq, sq), dtype=torch.float32, device=q.codes.device) if return_lse else None
    p = _PrefillParams(int(bool(causal)), float(softmax_scale), int(kv_tile), _RULES[p_rule],
                       float(p_qmax), int(bool(l_from_quantized)))
    dq, dk, dv = q.desc(), k.desc(), v.desc()
    _check(_lib.mxattn_prefill(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), ctypes.byref(p),
                               _ptr(out), _DT[out.dtype], _ptr(lse), _stream(q.codes)))
    return (out, lse) if return_lse else out


def prefill_hybrid(q, k, v, q_bf16, k_bf16, v_bf16, window, idx=None, n_sel=None, softmax_scale=0.0,
                   kv_tile=128, p_rule="ocp", p_qmax=UOS_QMAX, l_from_quantized=True,
                   out_dtype=torch.float32, return_lse=False, out=None):
    """Causal prefill with per-row bf16 keys under one softmax: the window of
    each query row and the selected keys idx [B,Hkv,max_sel] (ascending, the
    first n_sel [B,Hkv] of each row used) take the bf16 rows q_bf16
    [B,Hq,S,D], k_bf16/v_bf16 [B,Hkv,S,D]; every other key the MXFP4 path."""
    b, hq, sq, d = q.shape
    for t in (q_bf16, k_bf16, v_bf16):
        assert t.dtype == torch.bfloat16 and t.is_contiguous(), "bf16 rows must be contiguous bfloat16"
    if out is None:
        out = torch.empty((b, hq, sq, d), dtype=out_dtype, device=q.codes.device)
    lse = torch.empty((b, hq, sq), dtype=torch.float32, device=q.codes.device) if return_lse else None
    p = _PrefillParams(1, float(softmax_scale), int(kv_tile), _RULES[p_rule], float(p_qmax),
                       int(bool(l_from_quantized)))
    hy = _PrefillHybrid()
    hy.q, hy.k, hy.v = q_bf16.data_ptr(), k_bf16.data_ptr(), v_bf16.data_ptr()
    if idx is not None:
        assert idx.dtype == torch.int32 and idx.is_contiguous(), "idx must be contiguous int32"
        assert n_sel.dtype == torch.int32 and n_sel.is_contiguous(), "n_sel must be contiguous int32"
        hy.idx, hy.n_sel, hy.max_sel = idx.data_ptr(), n_sel.data_ptr(), idx.shape[-1]
    hy.window = int(window)
    dq, dk, dv = q.desc(), k.desc(), v.desc()
    _check(_lib.mxattn_prefill_hybrid(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), ctypes.byref(p),
                                      ctypes.byref(hy), _ptr(out), _DT[out.dtype], _ptr(lse), _stream(q.codes)))
    return (out, lse) if return_lse else out


def decode_workspace_bytes(batch, hq, hkv, dim, tcap, split_len, hybrid_rows=0):
    """Workspace of decode(); hybrid_rows = max_sel + window of the hybrid set."""
    return int(_lib.mxattn_decode_workspace_bytes(batch, hq, hkv, dim, tcap, split_len, int(hybrid_rows)))


def decode(q, k_cache, v_cache, ctx_len, softmax_scale=0.0, split_len=2048, hybrid=None,
           q_bf16=None, workspace=None, return_lse=False, out=None, q_res=None):
    """One query token per sequence against an MXFP4 KV cache.

    q: MX [B,Hq,1,D], or a bfloat16 tensor [B,Hq,D] / [B,Hq,1,D] that the scan
    encodes itself (OCP, the codes quantize() writes); caches: MX
    [B,Hkv,Tcap,D]; ctx_len int32 [B] on device.
    hybrid: None or dict(idx, n_sel, k_sel, v_sel, k_win, v_win, window).
    q_res: None or the residual MX of a dual-residual query (quantize_dual).
    """
    return _decode(q, k_cache, v_cache, None, k_cache.shape[2], ctx_len, softmax_scale, split_len, hybrid,
                   q_bf16, workspace, return_lse, out, q_res)


def decode_paged(q, k_pool, v_pool, block_table, ctx_len, softmax_scale=0.0, split_len=2048, hybrid=None,
                 q_bf16=None, workspace=None, return_lse=False, out=None, q_res=None):
    """decode() over a paged cache: k_pool/v_pool MX [n_pages,Hkv,page_size,D],
    block_table int32 [B,max_pages] (contiguous, on device) giving each
    sequence's physical pages in order."""
    assert block_table.dtype == torch.int32 and block_table.is_contiguous(), "block_table must be contiguous int32"
    pg = _Paging(block_table.data_ptr(), block_table.shape[1])
    return _decode(q, k_pool, v_pool, pg, block_table.shape[1] * k_pool.shape[2], ctx_len, softmax_scale,
                   split_len, hybrid, q_bf16, workspace, return_lse, out, q_res)


def _check_hybrid(hy, q_bf16, b, hq, hkv, d):
    """The C ABI receives the hybrid set as bare pointers: check here that
    each tensor has the dtype, layout and shape the scan reads."""
    def need(cond, what):
        if not cond:
            raise ValueError(f"decode hybrid: {what}")

    idx, n_sel = hy["idx"], hy["n_sel"]
    need(idx.dtype == torch.int32 and idx.is_contiguous() and idx.dim() == 3 and tuple(idx.shape[:2]) == (b, hkv),
         f"idx must be contiguous int32 [{b},{hkv},max_sel], got {idx.dtype} {tuple(idx.shape)}")
    need(n_sel.dtype == torch.int32 and n_sel.is_contiguous() and tuple(n_sel.shape) == (b, hkv),
         f"n_sel must be contiguous int32 [{b},{hkv}], got {n_sel.dtype} {tuple(n_sel.shape)}")
    w = int(hy["window"])
    rows = {"k_sel": idx.shape[-1], "v_sel": idx.shape[-1]}
    if w > 0:
        rows.update(k_win=w, v_win=w)
    for name, r in rows.items():
        t = hy.get(name)
        need(t is not None and t.dtype == torch.bfloat16 and t.is_contiguous() and tuple(t.shape) == (b, hkv, r, d),
             f"{name} must be contiguous bfloat16 [{b},{hkv},{r},{d}]"
             + ("" if t is None else f", got {t.dtype} {tuple(t.shape)}"))
    need(q_bf16 is not None and q_bf16.dtype == torch.bfloat16 and q_bf16.is_contiguous()
         and q_bf16.numel() == b * hq * d and q_bf16.shape[0] == b and q_bf16.shape[1] == hq,
         f"q_bf16 must be contiguous bfloat16 [{b},{hq},{d}]")


DECODE_SCRATCH_BYTES = 16 << 20   # the built-in scratch of decode_noalloc


def decode_noalloc(q, k_cache, v_cache, ctx_len, out, softmax_scale=0.0, split_len=2048, hybrid=None,
                   q_bf16=None, lse=None, q_res=None):
    """decode() through mxattn_decode_noalloc: no workspace, no allocation by
    the library or by this wrapper (out [B,Hq,D] fp32 and the optional lse
    [B,Hq] fp32 are the caller's).  The partial slots use the library's
    per-device scratch, so calls that overlap on one GPU race."""
    if out is None:
        raise ValueError("decode_noalloc: out must be given (the call allocates nothing)")
    return _decode(q, k_cache, v_cache, None, k_cache.shape[2], ctx_len, softmax_scale, split_len, hybrid,
                   q_bf16, None, lse is not None, out, q_res, noalloc=True, lse=lse)


def _decode(q, kc, vc, paging, tcap, ctx_len, softmax_scale, split_len, hybrid, q_bf16, workspace, return_lse,
            out, q_res, noalloc=False, lse=None):
    if isinstance(q, torch.Tensor):
        # bf16 query [B,Hq,D] or [B,Hq,1,D]: the scan encodes it (OCP), no
        # separate quantiser launch.
        assert q.dtype == torch.bfloat16, "an unencoded query must be bfloat16"
        qb = q.reshape(q.shape[0], q.shape[1], q.shape[-1]).contiguous()
        assert q_bf16 is None or q_bf16.data_ptr() == qb.data_ptr(), "pass the bf16 query once, as q"
        q_bf16 = qb
        q = MX(None, None, (qb.shape[0], qb.shape[1], 1, qb.shape[2]), "hd")
    b, hq, _, d = q.shape
    hkv = kc.shape[1]
    dev = kc.codes.device
    if hybrid is not None:
        _check_hybrid(hybrid, q_bf16, b, hq, hkv, d)
    hy_rows = (hybrid["idx"].shape[-1] + int(hybrid["window"])) if hybrid is not None else 0
    if not noalloc:
        need = decode_workspace_bytes(b, hq, hkv, d, tcap, split_len, hy_rows)
        if workspace is None or workspace.numel() < need:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if out is None:
        out = torch.empty((b, hq, d), dtype=torch.float32, device=dev)
    if return_lse and lse is None:
        lse = torch.empty((b, hq), dtype=torch.float32, device=dev)
    for t, shape in ((out, (b, hq, d)), (lse, (b, hq))):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != math.prod(shape)):
            raise ValueError(f"decode: out/lse must be contiguous float32 {shape}")
    hy = None
    if hybrid is not None:
        hy = _Hybrid()
        hy.idx, hy.n_sel = hybrid["idx"].data_ptr(), hybrid["n_sel"].data_ptr()
        hy.max_sel = hybrid["idx"].shape[-1]
        hy.window = int(hybrid["window"])
        hy.k_sel, hy.v_sel = hybrid["k_sel"].data_ptr(), hybrid["v_sel"].data_ptr()
        hy.k_win = hybrid["k_win"].data_ptr() if hybrid.get("k_win") is not None else None
        hy.v_win = hybrid["v_win"].data_ptr() if hybrid.get("v_win") is not None else None
    dq, dk, dv = q.desc(), kc.desc(), vc.desc()
    dqr = q_res.desc() if q_res is not None else None
    common = (ctypes.byref(dqr) if dqr is not None else None, _ptr(q_bf16), ctypes.byref(dk), ctypes.byref(dv))
    hyp = ctypes.byref(hy) if hy is not None else None
    if noalloc:
        _check(_lib.mxattn_decode_noalloc(ctypes.byref(dq), *common, _ptr(ctx_len), hyp, float(softmax_scale),
                                          int(split_len), _ptr(out), _ptr(lse), _stream(kc.codes)))
        return (out, lse) if return_lse else out
    tail = (_ptr(ctx_len), hyp, float(softmax_scale), int(split_len),
            _ptr(workspace), workspace.numel(), _ptr(out), _ptr(lse), _stream(kc.codes))
    if paging is None:
        _check(_lib.mxattn_decode(ctypes.byref(dq), *common, *tail))
    else:
        _check(_lib.mxattn_decode_paged(ctypes.byref(dq), *common, ctypes.byref(paging), *tail))
    return (out, lse) if return_lse else out


def select_workspace_bytes(batch, hq, recent, tcap):
    return int(_lib.mxattn_select_workspace_bytes(batch, hq, recent, tcap))


def select_vertical(q_recent, k_cache, ctx_len, col_mass, window, rho_num=5, rho_den=100,
                    max_sel=None, softmax_scale=0.0, workspace=None):
    """Accumulate column mass (in place) and select vertical-line tokens.

    Returns (idx int32 [B,Hkv,max_sel] ascending, n int32 [B,Hkv])."""
    b, hkv, tcap, d = k_cache.shape
    dev = k_cache.codes.device
    if max_sel is None:
        max_sel = max(-(-(tcap - window) * rho_num // rho_den), 1)
    hq = q_recent.shape[1] if q_recent is not None else hkv
    r = q_recent.shape[2] if q_recent is not None else 0
    need = select_workspace_bytes(b, hq, r, tcap)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    idx = torch.empty((b, hkv, max_sel), dtype=torch.int32, device=dev)
    n = torch.empty((b, hkv), dtype=torch.int32, device=dev)
    dq = q_recent.desc() if q_recent is not None else None
    dk = k_cache.desc()
    _check(_lib.mxattn_select_vertical(ctypes.byref(dq) if dq is not None else None, ctypes.byref(dk),
                                       _ptr(ctx_len), float(softmax_scale), int(window), int(rho_num),
                                       int(rho_den), _ptr(col_mass), _ptr(idx), _ptr(n), int(max_sel),
                                       _ptr(workspace), workspace.numel(), _stream(k_cache.codes)))
    return idx, n


def gather_rows(k, v, idx, n_sel, k_out=None, v_out=None):
    """bf16 rows of the selected tokens: k_out[b,h,i] = k[b,h,idx[b,h,i]] for
    i < n_sel[b,h] (k, v: bf16 [B,H,T,D] with contiguous channels; idx int32
    [B,H,max_sel], n_sel int32 [B,H]).  Returns (k_out, v_out), bf16
    [B,H,max_sel,D]; rows at or past n_sel are not written."""
    b, h, t, d = k.shape

    def need(cond, what):
        if not cond:
            raise ValueError(f"gather_rows: {what}")

    need(k.dtype == torch.bfloat16 and v.dtype == torch.bfloat16 and tuple(v.shape) == (b, h, t, d), "k, v bf16 [B,H,T,D]")
    need(k.stride(3) == 1 and v.stride(3) == 1, "channels must be contiguous")
    need(idx.dtype == torch.int32 and idx.is_contiguous() and idx.dim() == 3 and tuple(idx.shape[:2]) == (b, h),
         "idx contiguous int32 [B,H,max_sel]")
    need(n_sel.dtype == torch.int32 and n_sel.is_contiguous() and tuple(n_sel.shape) == (b, h), "n_sel int32 [B,H]")
    m = idx.shape[-1]
    if k_out is None:
        k_out = torch.empty((b, h, m, d), dtype=torch.bfloat16, device=k.device)
    if v_out is None:
        v_out = torch.empty((b, h, m, d), dtype=torch.bfloat16, device=k.device)
    for o in (k_out, v_out):
        need(o.dtype == torch.bfloat16 and o.is_contiguous() and tuple(o.shape) == (b, h, m, d), "outputs bf16 [B,H,max_sel,D]")
    shape = (ctypes.c_int64 * 4)(b, h, t, d)
    ks = (ctypes.c_int64 * 3)(k.stride(0), k.stride(1), k.stride(2))
    vs = (ctypes.c_int64 * 3)(v.stride(0), v.stride(1), v.stride(2))
    _check(_lib.mxattn_gather_rows(_ptr(k), _ptr(v), shape, ks, vs, _ptr(idx), _ptr(n_sel), int(m), _ptr(k_out),
                                   _ptr(v_out), _stream(k)))
    return k_out, v_out
