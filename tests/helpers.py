"""Test plumbing between torch tensors (GPU results, generator inputs) and the
numpy oracle.  Nothing here computes the method: the oracle does."""

import numpy as np
import torch

from oracle import attention, mx, rotate, smooth
from oracle import select as oracle_select


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


def check_prefill(q, k, v, qh, kh, vh, out, lse, *, causal, kv_tile=128, p_rule="ocp", qkv_rule="ocp",
                  l_from_quantized=True, rows=None, q_scale=None, k_scale=None, heads=None, what="",
                  hadamard=False, hybrid=None, q_rows_only=False, atol=2e-3):
    """Compare a finished GPU prefill with the oracle.

    q, k, v: the generator tensors; qh, kh, vh: the GPU's MXFP4 operands;
    out, lse: the GPU's results.  On query heads ``heads`` (default all) and
    rows ``rows`` (dict hq -> row indices, default all): the Q/K/V codes and
    scales bit for bit, then every row's output within atol plus the oracle's
    rounding envelope (8e-3 more for 16-bit outputs) and lse within 1e-3.
    With q_rows_only, only the sampled rows of Q are encoded by the oracle
    (rows are independent) and compared.  hybrid: dict(window, idx, n_sel)
    as passed to the GPU; the oracle reads the same selected positions."""
    bsz, hq = q.shape[0], q.shape[1]
    hkv = k.shape[1]
    grp = hq // hkv
    heads = list(range(hq)) if heads is None else list(heads)
    kv_heads = sorted({h // grp for h in heads})
    r = mx.RULE_OCP if qkv_rule == "ocp" else mx.RULE_UOS
    pr = mx.RULE_OCP if p_rule == "ocp" else mx.RULE_UOS
    ksel = torch.as_tensor(kv_heads, device=q.device)
    k32 = host_f64(k.index_select(1, ksel)).astype(np.float32)
    if k_scale is not None:
        k32 = smooth.apply(k32, k_scale.cpu().numpy()[kv_heads])
    if hadamard:
        k32 = rotate.hadamard_f32(k32, axis=3)
    ok = oracle_quantize(k32.astype(np.float64), "hd", r)
    ov = oracle_quantize(host_f64(v.index_select(1, ksel)), "key", r)
    assert_codes_equal(head_slice(kh, kv_heads), *ok, what + " k")
    assert_codes_equal(head_slice(vh, kv_heads), *ov, what + " v")
    kd = oracle_dequant(*ok, "hd")
    vd = oracle_dequant(*ov, "key", n=v.shape[2])
    del k32, ok, ov
    got = out.float().cpu().numpy()
    glse = lse.cpu().numpy()
    if out.dtype != torch.float32:
        atol = atol + 8e-3
    qc_all, qs_all = gpu_codes_unpacked(qh) if q_rows_only else (None, None)
    worst, n_env = 0.0, 0
    for i, h in enumerate(heads):
        rr = None if rows is None else np.asarray(rows[h])
        qsrc = q[:, h:h + 1]
        if q_rows_only and rr is not None:
            qsrc = qsrc.index_select(2, torch.as_tensor(rr, device=q.device))
        q32 = host_f64(qsrc).astype(np.float32)
        if q_scale is not None:
            q32 = smooth.apply(q32, q_scale.cpu().numpy()[[h]])
        if hadamard:
            q32 = rotate.hadamard_f32(q32, axis=3)
        oq = oracle_quantize(q32.astype(np.float64), "hd", r)
        if q_rows_only:
            gc, gs = qc_all[:, h:h + 1, rr], qs_all[:, h:h + 1, rr]
            assert np.array_equal(gs, oq[1]) and np.array_equal(gc, oq[0]), f"{what} q codes h{h}"
        else:
            assert_codes_equal(head_slice(qh, [h]), *oq, what + f" q h{h}")
        qd = oracle_dequant(*oq, "hd")
        kvi = kv_heads.index(h // grp)
        for bi in range(bsz):
            hy = None
            if hybrid is not None:
                kvh = h // grp
                sel = np.zeros(0, dtype=np.int64)
                if hybrid.get("idx") is not None:
                    sel = np.asarray(hybrid["idx"][bi, kvh, :int(hybrid["n_sel"][bi, kvh])].cpu())
                hy = {"window": hybrid["window"], "sel": sel, "q": host_f64(q[bi, h]),
                      "k": host_f64(k[bi, kvh]), "v": host_f64(v[bi, kvh])}
            qrow = qd[bi, 0]
            orows = rr
            if q_rows_only and rr is not None:
                # Only the sampled rows were encoded: scatter them back in place.
                full = np.zeros((q.shape[2], qd.shape[-1]))
                full[rr] = qrow
                qrow = full
            res = attention.prefill_head(qrow, kd[bi, kvi], vd[bi, kvi], causal=causal, kv_tile=kv_tile,
                                         p_rule=pr, l_from_quantized=l_from_quantized, rows=orows,
                                         envelope=True, hybrid=hy)
            g_rows = got[bi, h] if rr is None else got[bi, h][rr]
            l_rows = glse[bi, h] if rr is None else glse[bi, h][rr]
            worst = max(worst, check_within(g_rows, res["out"], res["bound"], atol, f"{what} b{bi} h{h}"))
            n_env += int((res["bound"] > 0).sum())
            np.testing.assert_allclose(l_rows, res["lse"], atol=1e-3, rtol=0)
    print(f"  {what}: worst |err| {worst:.3e}; rows needing the envelope: {n_env}", flush=True)
    return worst


def check_selection(gpu_idx, gpu_n, oracle_cm, ctx, window, num, den, what):
    """A GPU top-k against the oracle's column mass: the count exact, the
    indices ascending and valid, every token clearly above the k-th mass
    present and none clearly below it (float masses may order near-ties
    either way)."""
    k, nn = oracle_select.n_select(ctx, window, num, den)
    assert gpu_n == k, f"{what}: count {gpu_n} vs {k}"
    cm = oracle_cm[:nn]
    order = np.sort(cm)[::-1]
    tau = order[k - 1]
    eps = 1e-4 * max(order[0], 1e-30)
    got = set(gpu_idx.tolist())
    assert len(got) == k and all(0 <= t < nn for t in got)
    assert np.all(np.diff(gpu_idx) > 0), "indices must be ascending"
    sure_in = set(np.nonzero(cm > tau + eps)[0].tolist())
    assert sure_in <= got, f"{what}: {len(sure_in - got)} clearly heavier tokens missing"
    assert all(cm[t] >= tau - eps for t in got), f"{what}: a clearly lighter token was selected"
