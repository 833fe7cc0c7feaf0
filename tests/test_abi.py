"""The C ABI on the host (no GPU needed): the library loads, exports every
symbol include/mxattn.h declares, and rejects bad arguments with a status and
a message before any launch; the fault-injection hook works."""

import ctypes
import os
import re

import pytest

import bit_microscaled_flashattention_amd as mxa

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "mxattn.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mxattn_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) >= 9
    lib = mxa.library()
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(mxa.EXPORTS) == names


def test_status_strings_and_version():
    lib = mxa.library()
    for code, word in ((0, b"ok"), (1, b"invalid"), (2, b"unsupported"), (3, b"workspace"), (4, b"HIP")):
        assert word in lib.mxattn_status_string(code)
    assert b"gfx950" in lib.mxattn_version()


def _mx(codes=16, scales=16, b=1, h=1, s=128, d=128, layout=0):
    m = mxa._Mx()
    m.codes, m.scales = codes, scales
    m.batch, m.heads, m.seq, m.dim = b, h, s, d
    m.layout = layout
    if layout == 0:
        rc, rs = d // 2, d // 32
        m.code_stride[:] = [h * s * rc, s * rc, rc]
        m.scale_stride[:] = [h * s * rs, s * rs, rs]
    else:
        nb = (s + 31) // 32
        m.code_stride[:] = [h * d * nb * 16, d * nb * 16, nb * 16]
        m.scale_stride[:] = [h * d * nb, d * nb, nb]
    return m


def _prefill(q, k, v, **kw):
    lib = mxa.library()
    p = mxa._PrefillParams(kw.get("causal", 0), kw.get("scale", 0.0), kw.get("kv_tile", 128),
                           kw.get("p_rule", 0), kw.get("p_qmax", 7.25), 1)
    return lib.mxattn_prefill(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), ctypes.byref(p),
                              ctypes.c_void_p(kw.get("out", 4096)), 0, None, None)


@pytest.mark.parametrize("case, status", [
    ("d96", mxa.ERR_UNSUPPORTED),
    ("null_codes", mxa.ERR_INVALID_ARG),
    ("misaligned_codes", mxa.ERR_INVALID_ARG),
    ("v_not_key_layout", mxa.ERR_UNSUPPORTED),
    ("gqa_mismatch", mxa.ERR_INVALID_ARG),
    ("causal_rect", mxa.ERR_UNSUPPORTED),
    ("kv_tile_96", mxa.ERR_UNSUPPORTED),
    ("uos_qmax_9", mxa.ERR_UNSUPPORTED),
    ("neg_scale", mxa.ERR_INVALID_ARG),
    ("out_misaligned", mxa.ERR_INVALID_ARG),
    ("short_row_stride", mxa.ERR_INVALID_ARG),
    ("k_head_2gib", mxa.ERR_UNSUPPORTED),
    ("k_scales_2gib", mxa.ERR_UNSUPPORTED),
    ("v_head_2gib", mxa.ERR_UNSUPPORTED),
])
def test_prefill_rejects(case, status):
    q, k, v = _mx(), _mx(), _mx(layout=1)
    kw = {}
    if case == "d96":
        q, k, v = _mx(d=96), _mx(d=96), _mx(d=96, layout=1)
    elif case == "null_codes":
        q.codes = None
    elif case == "misaligned_codes":
        k.codes = 24
    elif case == "v_not_key_layout":
        v = _mx()
    elif case == "gqa_mismatch":
        q = _mx(h=3); k = _mx(h=2); v = _mx(h=2, layout=1)
    elif case == "causal_rect":
        q = _mx(s=64); kw["causal"] = 1
    elif case == "kv_tile_96":
        kw["kv_tile"] = 96
    elif case == "uos_qmax_9":
        kw["p_rule"], kw["p_qmax"] = 1, 9.0
    elif case == "neg_scale":
        kw["scale"] = -1.0
    elif case == "out_misaligned":
        kw["out"] = 4100
    elif case == "short_row_stride":
        k.code_stride[2] = 32
    elif case in ("k_head_2gib", "k_scales_2gib"):
        # 512K keys in rows of 4 KiB codes (or 4 KiB scales): one K head spans 2 GiB.
        s = 1 << 19
        q, k, v = _mx(s=s), _mx(s=s), _mx(s=s, layout=1)
        for t in (q, k):
            t.code_stride[:] = [4096 * s, 4096 * s, 4096] if case == "k_head_2gib" else [64 * s, 64 * s, 64]
            t.scale_stride[:] = [4096 * s, 4096 * s, 4096] if case == "k_scales_2gib" else [4 * s, 4 * s, 4]
    elif case == "v_head_2gib":
        # 128 channel rows of 16 MiB: one V head spans 2 GiB.
        v.code_stride[:] = [128 << 24, 128 << 24, 1 << 24]
    st = _prefill(q, k, v, **kw)
    assert st == status
    assert len(mxa.library().mxattn_last_error()) > 0
    if case.endswith("2gib"):
        assert b"2 GiB" in mxa.library().mxattn_last_error()


@pytest.mark.parametrize("case, status", [
    ("null_set", mxa.ERR_INVALID_ARG),
    ("not_causal", mxa.ERR_UNSUPPORTED),
    ("too_long", mxa.ERR_UNSUPPORTED),
    ("null_rows", mxa.ERR_INVALID_ARG),
    ("misaligned_rows", mxa.ERR_INVALID_ARG),
    ("neg_window", mxa.ERR_INVALID_ARG),
    ("neg_max_sel", mxa.ERR_INVALID_ARG),
    ("null_idx", mxa.ERR_INVALID_ARG),
    ("d96", mxa.ERR_UNSUPPORTED),
])
def test_prefill_hybrid_rejects(case, status):
    """Argument checks of mxattn_prefill_hybrid, all taken before any launch."""
    lib = mxa.library()
    q, k, v = _mx(), _mx(), _mx(layout=1)
    hy = mxa._PrefillHybrid()
    hy.q, hy.k, hy.v = 4096, 8192, 12288
    hy.idx, hy.n_sel, hy.max_sel, hy.window = 16384, 20480, 8, 64
    causal = 1
    if case == "not_causal":
        causal = 0
    elif case == "too_long":
        q, k, v = _mx(s=65537), _mx(s=65537), _mx(s=65537, layout=1)
    elif case == "null_rows":
        hy.v = None
    elif case == "misaligned_rows":
        hy.k = 8200
    elif case == "neg_window":
        hy.window = -1
    elif case == "neg_max_sel":
        hy.max_sel = -2
    elif case == "null_idx":
        hy.idx = None
    elif case == "d96":
        q, k, v = _mx(d=96), _mx(d=96), _mx(d=96, layout=1)
    p = mxa._PrefillParams(causal, 0.0, 128, 0, 7.25, 1)
    st = lib.mxattn_prefill_hybrid(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), ctypes.byref(p),
                                   None if case == "null_set" else ctypes.byref(hy),
                                   ctypes.c_void_p(4096), 0, None, None)
    assert st == status, mxa.library().mxattn_last_error()
    assert len(mxa.library().mxattn_last_error()) > 0


@pytest.mark.parametrize("shape, status", [
    ((0, 1, 128, 128), mxa.ERR_INVALID_ARG), ((1, 0, 128, 128), mxa.ERR_INVALID_ARG),
    ((1, 1, 0, 128), mxa.ERR_INVALID_ARG), ((65536, 1, 32, 128), mxa.ERR_UNSUPPORTED),
    ((1, 65536, 32, 128), mxa.ERR_UNSUPPORTED), ((1, 1, (1 << 26) + 32, 64), mxa.ERR_UNSUPPORTED),
    ((1, 1, 128, 256), mxa.ERR_UNSUPPORTED),
])
def test_empty_and_oversized_shapes_rejected(shape, status):
    """Empty tensors and shapes past the grid limits are refused by every
    entry point before any launch."""
    lib = mxa.library()
    b, h, s, d = shape
    q, k, v = _mx(b=b, h=h, s=s, d=d), _mx(b=b, h=h, s=s, d=d), _mx(b=b, h=h, s=s, d=d, layout=1)
    assert _prefill(q, k, v) == status
    strides = (ctypes.c_int64 * 3)(h * s * d, s * d, d)
    assert lib.mxattn_quantize(ctypes.c_void_p(4096), 2, strides, None, 0, 7.25, 0, ctypes.byref(q), None) == status
    q1 = _mx(b=b, h=h, s=1, d=d) if s != 0 else _mx(b=b, h=h, s=0, d=d)
    st = lib.mxattn_decode(ctypes.byref(q1), None, None, ctypes.byref(k), ctypes.byref(k), ctypes.c_void_p(64), None,
                           0.0, 2048, ctypes.c_void_p(4096), 1 << 40, ctypes.c_void_p(4096), None, None)
    assert st == status, lib.mxattn_last_error()


def test_quantize_rejects_without_launch():
    lib = mxa.library()
    out = _mx()
    strides = (ctypes.c_int64 * 3)(0, 0, 128)
    assert lib.mxattn_quantize(None, 2, strides, None, 0, 7.25, 0, ctypes.byref(out), None) == mxa.ERR_INVALID_ARG
    assert lib.mxattn_quantize(ctypes.c_void_p(64), 7, strides, None, 0, 7.25, 0, ctypes.byref(out), None) == mxa.ERR_INVALID_ARG
    assert lib.mxattn_quantize(ctypes.c_void_p(64), 2, strides, None, 1, 8.5, 0, ctypes.byref(out), None) == mxa.ERR_UNSUPPORTED
    assert lib.mxattn_quantize(ctypes.c_void_p(65), 2, strides, None, 0, 7.25, 0, ctypes.byref(out), None) == mxa.ERR_INVALID_ARG


def test_quantize_flags_rejects_without_launch():
    lib = mxa.library()
    strides = (ctypes.c_int64 * 3)(0, 0, 128)
    out, kout = _mx(), _mx(layout=1)
    x = ctypes.c_void_p(64)
    assert lib.mxattn_quantize(x, 2, strides, None, 0, 7.25, 4, ctypes.byref(out), None) == mxa.ERR_INVALID_ARG
    assert b"flags" in lib.mxattn_last_error()
    assert lib.mxattn_quantize(x, 2, strides, None, 0, 7.25, mxa.QUANT_HADAMARD, ctypes.byref(kout), None) == \
        mxa.ERR_UNSUPPORTED
    assert b"Hadamard" in lib.mxattn_last_error()


def test_quantize_batch_rejects_without_launch():
    lib = mxa.library()
    outs = [_mx(), _mx(layout=1)]
    jobs = (mxa._QuantJob * 5)()
    for j in jobs:
        j.x = 64
        j.x_dtype = 2
        j.x_stride[:] = [0, 0, 128]
        j.rule = 0
        j.qmax = 7.25
        j.out = ctypes.pointer(outs[0])
    assert lib.mxattn_quantize_batch(None, 1, None) == mxa.ERR_INVALID_ARG
    assert lib.mxattn_quantize_batch(jobs, 0, None) == mxa.ERR_INVALID_ARG
    assert lib.mxattn_quantize_batch(jobs, 5, None) == mxa.ERR_INVALID_ARG
    # A bad later job stops the whole batch and is named in the message.
    jobs[1].rule, jobs[1].qmax = 1, 8.5
    assert lib.mxattn_quantize_batch(jobs, 2, None) == mxa.ERR_UNSUPPORTED
    assert b"job[1]" in lib.mxattn_last_error()
    jobs[1].rule, jobs[1].qmax = 0, 7.25
    jobs[1].out = ctypes.pointer(outs[1])
    jobs[1].x = 66
    assert lib.mxattn_quantize_batch(jobs, 2, None) == mxa.ERR_INVALID_ARG
    assert b"job[1]" in lib.mxattn_last_error()
    jobs[0].out = None
    assert lib.mxattn_quantize_batch(jobs, 1, None) == mxa.ERR_INVALID_ARG


def test_calibrate_rejects():
    lib = mxa.library()
    f = ctypes.c_void_p(64)
    assert lib.mxattn_smooth_calibrate(f, f, 2, 6, 4, 16, 128, f, f, None) == mxa.ERR_INVALID_ARG
    assert lib.mxattn_smooth_calibrate(f, f, 2, 8, 4, 16, 512, f, f, None) == mxa.ERR_UNSUPPORTED
    assert lib.mxattn_smooth_calibrate(None, f, 2, 8, 4, 16, 128, f, f, None) == mxa.ERR_INVALID_ARG


def test_decode_workspace_and_rejects():
    lib = mxa.library()
    n = mxa.decode_workspace_bytes(32, 32, 8, 128, 32768, 2048)
    assert n == 32 * 32 * 16 * 130 * 4
    nh = mxa.decode_workspace_bytes(8, 32, 8, 128, 32768, 2048, hybrid_rows=1632 + 128)
    assert nh == 8 * 32 * (16 + 4) * 130 * 4      # bf16 set in parts of 512 rows
    assert mxa.decode_workspace_bytes(0, 32, 8, 128, 32768, 2048) == 0
    q = _mx(s=1, h=32); kc = _mx(s=32768, h=8); vc = _mx(s=32768, h=8)
    ctx = ctypes.c_void_p(64)
    out = ctypes.c_void_p(4096)
    # workspace too small
    st = lib.mxattn_decode(ctypes.byref(q), None, None, ctypes.byref(kc), ctypes.byref(vc), ctx, None, 0.0, 2048,
                           ctypes.c_void_p(4096), 16, out, None, None)
    assert st == mxa.ERR_WORKSPACE
    # split_len not a multiple of 64
    st = lib.mxattn_decode(ctypes.byref(q), None, None, ctypes.byref(kc), ctypes.byref(vc), ctx, None, 0.0, 100,
                           ctypes.c_void_p(4096), 1 << 30, out, None, None)
    assert st == mxa.ERR_UNSUPPORTED
    # group of 3 query heads per KV head
    q3 = _mx(s=1, h=24)
    st = lib.mxattn_decode(ctypes.byref(q3), None, None, ctypes.byref(kc), ctypes.byref(vc), ctx, None, 0.0, 2048,
                           ctypes.c_void_p(4096), 1 << 30, out, None, None)
    assert st == mxa.ERR_UNSUPPORTED
    # hybrid without a bf16 query
    hy = mxa._Hybrid()
    hy.max_sel, hy.window = 16, 8
    st = lib.mxattn_decode(ctypes.byref(q), None, None, ctypes.byref(kc), ctypes.byref(vc), ctx, ctypes.byref(hy),
                           0.0, 2048, ctypes.c_void_p(4096), 1 << 30, out, None, None)
    assert st == mxa.ERR_INVALID_ARG
    # residual query of another shape
    qr = _mx(s=1, h=16)
    st = lib.mxattn_decode(ctypes.byref(q), ctypes.byref(qr), None, ctypes.byref(kc), ctypes.byref(vc), ctx, None,
                           0.0, 2048, ctypes.c_void_p(4096), 1 << 30, out, None, None)
    assert st == mxa.ERR_INVALID_ARG
    assert b"q_res" in lib.mxattn_last_error()


@pytest.mark.parametrize("case, status", [
    ("null_paging", mxa.ERR_INVALID_ARG),
    ("null_table", mxa.ERR_INVALID_ARG),
    ("no_pages", mxa.ERR_INVALID_ARG),
    ("page_48", mxa.ERR_UNSUPPORTED),
    ("split_not_pages", mxa.ERR_UNSUPPORTED),
    ("split_65_pages", mxa.ERR_UNSUPPORTED),
    ("pools_differ", mxa.ERR_INVALID_ARG),
    ("capacity_overflow", mxa.ERR_UNSUPPORTED),
    ("workspace_small", mxa.ERR_WORKSPACE),
])
def test_decode_paged_rejects(case, status):
    """Argument checks of mxattn_decode_paged, all taken before any launch."""
    lib = mxa.library()
    q = _mx(s=1, h=32, b=4)
    kp, vp = _mx(b=100, h=8, s=64), _mx(b=100, h=8, s=64)
    pg = mxa._Paging(8192, 512)  # 512 pages of 64 tokens per sequence
    split = 2048
    ws = 1 << 30
    if case == "page_48":
        kp, vp = _mx(b=100, h=8, s=48), _mx(b=100, h=8, s=48)
    elif case == "null_table":
        pg.block_table = None
    elif case == "no_pages":
        pg.max_pages = 0
    elif case == "split_not_pages":  # 2112 tokens: a multiple of 64, not of the 128-token page
        kp, vp = _mx(b=100, h=8, s=128), _mx(b=100, h=8, s=128)
        split = 2112
    elif case == "split_65_pages":
        split = 65 * 64
    elif case == "pools_differ":
        vp = _mx(b=99, h=8, s=64)
    elif case == "capacity_overflow":
        pg.max_pages = (1 << 31) // 64
    elif case == "workspace_small":
        ws = 64
    st = lib.mxattn_decode_paged(ctypes.byref(q), None, None, ctypes.byref(kp), ctypes.byref(vp),
                                 None if case == "null_paging" else ctypes.byref(pg), ctypes.c_void_p(64), None,
                                 0.0, split, ctypes.c_void_p(4096), ws, ctypes.c_void_p(4096), None, None)
    assert st == status, mxa.library().mxattn_last_error()
    assert len(mxa.library().mxattn_last_error()) > 0


def test_quantize_dual_rejects_without_launch():
    lib = mxa.library()
    strides = (ctypes.c_int64 * 3)(0, 0, 128)
    out, res = _mx(), _mx()
    x = ctypes.c_void_p(64)
    # KEY layout
    kout = _mx(layout=1)
    assert lib.mxattn_quantize_dual(x, 2, strides, None, 0, 7.25, 0, ctypes.byref(kout), ctypes.byref(res), None) == \
        mxa.ERR_UNSUPPORTED
    # shapes differ
    res2 = _mx(s=65)
    assert lib.mxattn_quantize_dual(x, 2, strides, None, 0, 7.25, 0, ctypes.byref(out), ctypes.byref(res2), None) == \
        mxa.ERR_INVALID_ARG
    # null residual descriptor
    assert lib.mxattn_quantize_dual(x, 2, strides, None, 0, 7.25, 0, ctypes.byref(out), None, None) == mxa.ERR_INVALID_ARG


def test_select_rejects():
    lib = mxa.library()
    kc = _mx(s=32768, h=8)
    q = _mx(s=65, h=32)
    f = ctypes.c_void_p(4096)
    args = lambda qq, max_sel, ws: (ctypes.byref(qq) if qq else None, ctypes.byref(kc), f, 0.0, 128, 5, 100,
                                    f, f, f, max_sel, f, ws, None)
    assert lib.mxattn_select_vertical(*args(q, 4096, 1 << 30)) == mxa.ERR_UNSUPPORTED    # R > 64
    q = _mx(s=64, h=32)
    assert lib.mxattn_select_vertical(*args(q, 100, 1 << 30)) == mxa.ERR_INVALID_ARG     # max_sel too small
    assert lib.mxattn_select_vertical(*args(q, 1632, 8)) == mxa.ERR_WORKSPACE


def test_fault_injection(monkeypatch):
    q, k, v = _mx(), _mx(), _mx(layout=1)
    monkeypatch.setenv("MXATTN_INJECT", "prefill:4")
    assert _prefill(q, k, v) == mxa.ERR_HIP
    assert b"injected" in mxa.library().mxattn_last_error()
    monkeypatch.setenv("MXATTN_INJECT", "decode:3")
    # A different entry point is unaffected (and fails its own validation).
    q.codes = None
    assert _prefill(q, k, v) == mxa.ERR_INVALID_ARG


def test_python_errors_raise():
    with pytest.raises(mxa.MxattnError) as ei:
        mxa._check(mxa.ERR_UNSUPPORTED)
    assert ei.value.status == mxa.ERR_UNSUPPORTED


C_PROGRAM = r"""
#include <stdio.h>
#include "mxattn.h"
int main(void) {
  const mxattn_prefill_params_t p = {1, 0.0f, 128, MXATTN_SCALE_OCP, 7.25f, 1};
  int64_t shape[4] = {1, 1, 32, 128};
  mxattn_mx_t m = {0};
  /* Refused on the host before any launch: null codes. */
  const mxattn_status_t st = mxattn_prefill(&m, &m, &m, &p, 0, MXATTN_F32, 0, 0);
  (void)shape;
  printf("%d|%s|%s|%zu\n", (int)st, mxattn_status_string(st), mxattn_version(),
         mxattn_decode_workspace_bytes(32, 32, 8, 128, 32768, 4096, 0));
  return 0;
}
"""


def test_header_is_plain_c_and_links(tmp_path):
    """include/mxattn.h compiles as strict C99 and a C program links against
    the library and calls it (host-side entry points only)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "abi.c"
    src.write_text(C_PROGRAM)
    exe = tmp_path / "abi"
    libdir = os.path.dirname(mxa.LIB_PATH)
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I",
                        os.path.dirname(HEADER), str(src), "-o", str(exe), "-L", libdir, "-l:libmxattn.so",
                        f"-Wl,-rpath,{libdir}"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stderr
    st, text, version, ws = out.stdout.strip().split("|")
    assert int(st) == 1 and "invalid" in text and "gfx950" in version
    assert int(ws) == mxa.decode_workspace_bytes(32, 32, 8, 128, 32768, 4096)


def test_decode_unencoded_query_rejects():
    """A query descriptor without codes needs q_bf16 and cannot carry a
    dual-residual half; both are refused on the host."""
    lib = mxa.library()
    q = _mx(codes=None, scales=None, b=2, h=8, s=1, d=128)
    k = _mx(b=2, h=2, s=256, d=128)
    out = ctypes.c_void_p(16)
    ctx = ctypes.c_void_p(16)
    ws = ctypes.c_void_p(256)
    st = lib.mxattn_decode(ctypes.byref(q), None, None, ctypes.byref(k), ctypes.byref(k), ctx, None, 0.0, 256,
                           ws, 1 << 20, out, None, None)
    assert st == 1 and b"q_bf16" in lib.mxattn_last_error()
    qr = _mx(b=2, h=8, s=1, d=128)
    st = lib.mxattn_decode(ctypes.byref(q), ctypes.byref(qr), ctypes.c_void_p(16), ctypes.byref(k), ctypes.byref(k),
                           ctx, None, 0.0, 256, ws, 1 << 20, out, None, None)
    assert st == 2 and b"dual" in lib.mxattn_last_error()


@pytest.mark.parametrize("case", ["idx_int64", "idx_shape", "nsel_shape", "ksel_fp16", "ksel_strided",
                                  "vwin_short", "qbf16_missing"])
def test_decode_hybrid_arguments_checked_in_binding(case):
    """The hybrid set reaches the C ABI as bare pointers, so the binding checks
    dtype, contiguity and shape of every tensor before anything is called
    (CPU tensors: a check that passed would reach the library and fail there
    with a different error)."""
    import torch
    b, hq, hkv, t, d, w, ms = 2, 8, 2, 256, 128, 16, 12
    cache = mxa.MX(torch.zeros((b, hkv, t, d // 2), dtype=torch.uint8),
                   torch.zeros((b, hkv, t, d // 32), dtype=torch.uint8), (b, hkv, t, d), "hd")
    q = mxa.MX(torch.zeros((b, hq, 1, d // 2), dtype=torch.uint8),
               torch.zeros((b, hq, 1, d // 32), dtype=torch.uint8), (b, hq, 1, d), "hd")
    bf = dict(dtype=torch.bfloat16)
    hy = {"idx": torch.zeros((b, hkv, ms), dtype=torch.int32), "n_sel": torch.zeros((b, hkv), dtype=torch.int32),
          "k_sel": torch.zeros((b, hkv, ms, d), **bf), "v_sel": torch.zeros((b, hkv, ms, d), **bf),
          "k_win": torch.zeros((b, hkv, w, d), **bf), "v_win": torch.zeros((b, hkv, w, d), **bf), "window": w}
    qb = torch.zeros((b, hq, d), **bf)
    if case == "idx_int64":
        hy["idx"] = hy["idx"].long()
    elif case == "idx_shape":
        hy["idx"] = torch.zeros((b, hq, ms), dtype=torch.int32)
    elif case == "nsel_shape":
        hy["n_sel"] = torch.zeros((b,), dtype=torch.int32)
    elif case == "ksel_fp16":
        hy["k_sel"] = hy["k_sel"].half()
    elif case == "ksel_strided":
        hy["k_sel"] = torch.zeros((b, hkv, d, ms), **bf).transpose(2, 3)
    elif case == "vwin_short":
        hy["v_win"] = torch.zeros((b, hkv, w - 1, d), **bf)
    elif case == "qbf16_missing":
        qb = None
    with pytest.raises(ValueError, match="decode hybrid"):
        mxa.decode(q, cache, cache, torch.full((b,), t, dtype=torch.int32), split_len=128, hybrid=hy, q_bf16=qb)


def test_decode_noalloc_refuses_problems_beyond_its_scratch():
    """The no-allocation decode checks that its partial slots fit the 16 MiB
    built-in scratch before it touches the device (here there is none: a
    check that passed would fail later with a different status)."""
    lib = mxa.library()
    b, hq, hkv, t = 64, 64, 16, 32768
    q, k = _mx(b=b, h=hq, s=1), _mx(b=b, h=hkv, s=t)
    need = lib.mxattn_decode_workspace_bytes(b, hq, hkv, 128, t, 2048, 0)
    assert need > mxa.DECODE_SCRATCH_BYTES
    st = lib.mxattn_decode_noalloc(ctypes.byref(q), None, None, ctypes.byref(k), ctypes.byref(k),
                                   ctypes.c_void_p(64), None, 0.0, 2048, ctypes.c_void_p(4096), None, None)
    assert st == mxa.ERR_UNSUPPORTED
    assert b"scratch" in lib.mxattn_last_error()
    # Argument errors come first, as for mxattn_decode.
    q.codes = None
    st = lib.mxattn_decode_noalloc(ctypes.byref(q), None, None, ctypes.byref(k), ctypes.byref(k),
                                   ctypes.c_void_p(64), None, 0.0, 2048, ctypes.c_void_p(4096), None, None)
    assert st == mxa.ERR_INVALID_ARG


def test_decode_noalloc_python_wrapper_needs_out():
    with pytest.raises(ValueError, match="out must be given"):
        mxa.decode_noalloc(None, None, None, None, None)


@pytest.mark.parametrize("bad", ["out_fp16", "out_shape", "lse_shape"])
def test_decode_output_checked_in_binding(bad):
    """out [B,Hq,D] and lse [B,Hq] must be contiguous float32 of those sizes;
    checked before the library is called (CPU tensors)."""
    import torch
    b, hq, hkv, t, d = 2, 8, 2, 256, 128
    cache = mxa.MX(torch.zeros((b, hkv, t, d // 2), dtype=torch.uint8),
                   torch.zeros((b, hkv, t, d // 32), dtype=torch.uint8), (b, hkv, t, d), "hd")
    q = mxa.MX(torch.zeros((b, hq, 1, d // 2), dtype=torch.uint8),
               torch.zeros((b, hq, 1, d // 32), dtype=torch.uint8), (b, hq, 1, d), "hd")
    out = torch.zeros((b, hq, d), dtype=torch.float16 if bad == "out_fp16" else torch.float32)
    if bad == "out_shape":
        out = torch.zeros((b, hq, d - 1))
    lse = torch.zeros((b, hq + (bad == "lse_shape")))
    with pytest.raises(ValueError, match="out/lse"):
        mxa.decode_noalloc(q, cache, cache, torch.full((b,), t, dtype=torch.int32), out, split_len=128, lse=lse)


def _gather(k=4096, v=8192, shape=(2, 4, 100, 128), ks=None, vs=None, idx=64, n=128, max_sel=16, ko=12288, vo=16384):
    lib = mxa.library()
    b, h, t, d = shape
    st = (ctypes.c_int64 * 4)(*shape)
    ks = (ctypes.c_int64 * 3)(*(ks or (h * t * d, t * d, d)))
    vs = (ctypes.c_int64 * 3)(*(vs or (h * t * d, t * d, d)))
    return lib.mxattn_gather_rows(ctypes.c_void_p(k), ctypes.c_void_p(v), st, ks, vs, ctypes.c_void_p(idx),
                                  ctypes.c_void_p(n), max_sel, ctypes.c_void_p(ko), ctypes.c_void_p(vo), None)


@pytest.mark.parametrize("kw, status", [
    (dict(shape=(2, 4, 100, 96)), mxa.ERR_UNSUPPORTED),
    (dict(shape=(0, 4, 100, 128)), mxa.ERR_INVALID_ARG),
    (dict(shape=(300, 300, 100, 128)), mxa.ERR_UNSUPPORTED),
    (dict(max_sel=-1), mxa.ERR_INVALID_ARG),
    (dict(k=4100), mxa.ERR_INVALID_ARG),
    (dict(vo=0), mxa.ERR_INVALID_ARG),
    (dict(ks=(51200, 12800, 100)), mxa.ERR_INVALID_ARG),
    (dict(vs=(51200, 12800, 64)), mxa.ERR_INVALID_ARG),
])
def test_gather_rows_rejects(kw, status):
    """Argument checks of mxattn_gather_rows, all on the host."""
    assert _gather(**kw) == status, mxa.library().mxattn_last_error()
    assert len(mxa.library().mxattn_last_error()) > 0


def test_gather_rows_zero_rows_is_a_no_op():
    assert _gather(max_sel=0, idx=0, n=0, ko=0, vo=0) == mxa.OK
