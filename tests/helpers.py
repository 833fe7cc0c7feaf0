"""Test plumbing between torch tensors (GPU results, generator inputs) and the
numpy oracle.  Nothing here computes the method: the oracle does."""

import numpy as np
import torch

from oracle import mx


def host_f64(t):
    """Exact float64 copy of a bf16/fp16/fp32 torch tensor."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def host_f32(t):
    return t.detach().to("cpu").to(torch.float32).numpy()


def gpu_codes_unpacked(m):
    """Unpacked GPU codes/scales of an MX tensor in the oracle's axis order.

    hd:  codes [B,H,S,D], scales [B,H,S,D/32]
    key: codes [B,H,S_pad,D], scales [B,H,S_pad/32,D]
    """
    c = mx.unpack_nibbles(m.codes.to("cpu").numpy(), axis=-1)
    s = m.scales.to("cpu").numpy()
    if m.layout == "key":
        c = np.swapaxes(c, 2, 3)
        s = np.swapaxes(s, 2, 3)
    return c, s


def oracle_quantize(x32, layout, rule=mx.RULE_OCP, qmax=mx.UOS_QMAX):
    """Oracle codes/scales of float values x32 [B,H,S,D] (hd: blocks on D,
    key: blocks on S), in the axis order of gpu_codes_unpacked.  Heads are
    processed one at a time to bound host memory."""
    axis = 3 if layout == "hd" else 2
    cs, ss = [], []
    for h in range(x32.shape[1]):
        c, s = mx.quantize(x32[:, h:h + 1], axis=axis, rule=rule, qmax=qmax)
        cs.append(c)
        ss.append(s)
    return np.concatenate(cs, axis=1), np.concatenate(ss, axis=1)


def head_slice(m, heads):
    """The MX tensor restricted to a list of heads (a gathered copy)."""
    idx = torch.as_tensor(heads, device=m.codes.device)
    return type(m)(m.codes.index_select(1, idx), m.scales.index_select(1, idx),
                   (m.shape[0], len(heads), m.shape[2], m.shape[3]), m.layout)


def oracle_dequant(codes, scales, layout, n=None):
    axis = 3 if layout == "hd" else 2
    return mx.dequantize(codes, scales, axis=axis, n=n)


def assert_codes_equal(gpu_mx, oracle_codes, oracle_scales, what=""):
    gc, gs = gpu_codes_unpacked(gpu_mx)
    if gpu_mx.layout == "key":
        # The GPU stores the padded tail; compare the blocks the oracle has.
        gc = gc[:, :, :oracle_codes.shape[2]]
        gs = gs[:, :, :oracle_scales.shape[2]]
    bad_s = np.argwhere(gs != oracle_scales)
    assert bad_s.shape[0] == 0, f"{what}: {bad_s.shape[0]} scale bytes differ, first at {bad_s[:3].tolist()}"
    bad_c = np.argwhere(gc != oracle_codes)
    assert bad_c.shape[0] == 0, f"{what}: {bad_c.shape[0]} codes differ, first at {bad_c[:3].tolist()}"


def check_within(gpu, ref, bound, atol=2e-3, what=""):
    """|gpu - ref| <= atol + bound row-wise (bound: per-row rounding envelope)."""
    err = np.abs(np.asarray(gpu, np.float64) - ref).max(axis=-1)
    lim = atol + (bound if bound is not None else 0.0)
    bad = np.argwhere(err > lim)
    assert bad.shape[0] == 0, (f"{what}: {bad.shape[0]} rows over tolerance; worst err "
                               f"{err.max():.3e}, first {bad[:3].tolist()}")
    return float(err.max())
