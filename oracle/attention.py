"""MXFP4 attention forward: tiled prefill with pre-normalisation P quantisation,
and the fused-dequantisation decode softmax over an MXFP4 (optionally hybrid)
KV set.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources
  * HiFA4 page, Abstract: QK^T and PV both run on 4-bit operands; the online
    softmax state is kept in higher precision; P-Reordering accumulates the
    softmax normaliser from the same quantised weights P_hat that enter the PV
    product, instead of from a higher-precision reconstruction.
  * MXAttention page, Abstract: Pre-Normalization Quantization quantises the
    unnormalised softmax exponentials before the row-wise summation, which
    keeps the normalisation exact by construction; UOS bounds the scales.
  * BitDecoding-FP4 page, "System-Level Optimization": P is quantised in
    place during the block-wise softmax and never written to memory.
  * HyQuant page (method paragraphs): one online softmax across 4-bit tokens
    and the full-precision vertical-line and window tokens; in decode the
    4-bit cache is dequantised inside the scan.

The operands handed to these functions are already-dequantised float64
arrays (q_hat, k_hat, v_hat).  Quantisation of Q, K, V is done separately with
oracle.mx so that each step can be checked on its own.

Readings
  * softmax_scale (1/sqrt(D) by default) multiplies the logits after the
    product; it is not folded into Q before quantisation.
  * Keys are visited in tiles of Bc = kv_tile keys in ascending order.  The
    reference maximum for the exponentials of a tile is the running maximum
    after that tile has been seen (the FlashAttention-2 update), so P_hat
    depends on Bc and on the order; the oracle takes Bc as a parameter.
  * P is quantised per (query row, 32 consecutive keys), blocks aligned to the
    tile start; masked or out-of-range keys contribute 0 and never raise a
    block maximum.  A tile with no visible key for a row leaves that row's
    state untouched.
  * Causal masking (Sq == Sk only): key t is visible to query i iff t <= i.
  * l_from_quantized=True is the PNQ / P-Reordering normaliser (l = sum P_hat);
    False is the baseline that sums the unquantised exponentials.
  * Hybrid prefill (HyQuant: in prefill the 4-bit and the full-precision
    tokens share one FlashAttention kernel and one online softmax).  Query i
    uses the full-precision rows for its ``window`` most recent keys
    (i - window < t <= i) and for the selected vertical-line keys t <= i;
    every other visible key takes the 4-bit path.  The page fixes neither the
    prefill window nor the order of the two parts; the reading is a window
    that slides with the query (the decode window is the last tokens of the
    context) and the 4-bit tiles first, with the full-precision keys removed
    from them (they contribute 0 and never raise a P block maximum), then
    one update over all full-precision keys with P unquantised (l adds the
    unquantised exponentials).  So no 4-bit P quantisation decision depends
    on a full-precision logit.
  * Decode does not quantise P (none of the sources gives a decode P format; the
    cache's V blocks run along head_dim, so a 4-bit PV contraction over keys
    has no block scales to use).

Parity: pinned by tests/test_oracle_attention.py -- with quantisation off the
tiled prefill equals textbook softmax attention for every tile width; with a
tile wider than the sequence it equals a direct whole-row PNQ computation;
the effective weights are non-negative and sum to one per row; l >= 1; the
smoothing rescale is output-neutral; decode equals the prefill path on the
same operands; hybrid decode reduces to pure-FP4 and to pure-BF16 attention
in its two limits; hybrid prefill reduces to the 4-bit prefill (empty set,
window 0) and to textbook attention on the full-precision rows (window >= Sq),
equals textbook attention for any window and set when P is not quantised and
both operand sets coincide (every key counted once), and matches a direct
whole-row computation when one tile spans the sequence.  Across tiles, the
hand-worked two-tile table tests/golden/two_tile_running_max.txt fixes the
reference maximum (the running one, after the tile), the rescale of earlier
tiles and both normaliser rules under both scale rules.  The multi-head
wrappers prefill and decode are pinned against the repeat-each-KV-head form
of grouped-query attention (np.repeat along the head axis) with textbook
softmax, the direct whole-row PNQ and substituted hybrid rows.  Attention
values under quantisation on general inputs have no worked example in the
sources: beyond those cases and invariants they rest on the steps above.
"""

import numpy as np

from . import mx

# Envelope of float32 disagreement used when a GPU result is compared with
# this float64 oracle: an exponential computed in float32 from float32 logits
# is within relative  ETA0 + ETA1 * (|s| + |m|)  of the exact one (s, m in
# natural-log units).  A P element (or a block maximum) whose exact value lies
# that close to an E2M1 rounding midpoint (or a scale boundary) has two
# correct codes; the oracle reports how far the output can move if the other
# one is taken.
ETA0 = 2.0 ** -20
ETA1 = 2.0 ** -19

_MIDPOINTS = (mx.E2M1_VALUES[:-1] + mx.E2M1_VALUES[1:]) / 2.0


def _alt_code_step(z, eta):
    """For magnitudes z (in scale units) return the value change if rounding
    went to the other side of a midpoint lying within relative eta of z
    (0 where no midpoint is that close)."""
    step = np.zeros_like(z)
    for k, mid in enumerate(_MIDPOINTS):
        near = np.abs(z - mid) <= eta * mid
        step = np.where(near, mx.E2M1_VALUES[k + 1] - mx.E2M1_VALUES[k], step)
    return step


def _quantize_p_rows(pt, rule, qmax):
    """Quantise rows of unnormalised exponentials in 32-key blocks.

    pt: [R, n] with n a multiple of 32.  Returns (P_hat [R, n], e [R, n/32]).
    """
    codes, sb = mx.quantize_blocks(pt, rule, qmax)
    return mx.dequantize_blocks(codes, sb), sb.astype(np.int64) - 127


def _envelope_tile(pt, ph, e, s, m_new, rule, qmax):
    """Sum over a tile of |P_hat change| under every alternative rounding."""
    r, n = pt.shape
    eta = ETA0 + ETA1 * (np.abs(s) + np.abs(m_new)[:, None])
    eta = np.where(np.isfinite(eta), eta, 0.0)
    scale = np.ldexp(1.0, np.repeat(e, mx.BLOCK, axis=1))
    z = pt / scale
    delta = (_alt_code_step(z, eta) * scale).sum(axis=1)
    # Block maxima near a scale boundary: the whole block may be coded with
    # the neighbouring exponent.  A block whose maximum is exactly 1 (it holds
    # the running maximum itself) is exact on both sides and is skipped.
    blk = pt.reshape(r, n // mx.BLOCK, mx.BLOCK)
    amax = blk.max(axis=2)
    eta_b = eta.reshape(r, n // mx.BLOCK, mx.BLOCK).max(axis=2)
    if rule == mx.RULE_OCP:
        bound = np.ldexp(1.0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))).astype(np.int64))
        cand = [bound, 2.0 * bound]
    else:
        ee = mx.e8m0_exponent(amax, rule, qmax)
        cand = [qmax * np.ldexp(1.0, ee), qmax * np.ldexp(1.0, ee - 1)]
    near = np.zeros(amax.shape, dtype=bool)
    for b in cand:
        near |= np.abs(amax - b) <= eta_b * b
    near &= (amax > 0) & (amax != 1.0)
    if near.any():
        ph_blk = ph.reshape(r, n // mx.BLOCK, mx.BLOCK)
        for (i, bidx) in zip(*np.nonzero(near)):
            y = blk[i, bidx]
            e0 = e[i, bidx]
            for alt in (e0 - 1, e0 + 1):
                zz = np.ldexp(y, -alt)
                cz = mx.e2m1_round_magnitude(zz)
                alt_vals = np.ldexp(mx.E2M1_VALUES[cz], alt)
                delta[i] += np.abs(alt_vals - ph_blk[i, bidx]).sum()
    return delta


def prefill_head(q, k, v, *, causal=False, softmax_scale=None, kv_tile=128,
                 quantize_p=True, p_rule=mx.RULE_OCP, p_qmax=mx.UOS_QMAX,
                 l_from_quantized=True, rows=None, envelope=False,
                 return_weights=False, return_tile_eps=False, hybrid=None, _perturb=None):
    """One head of the tiled online-softmax forward pass.

    q: [Sq, D], k/v: [Sk, D] float64 (dequantised operands or raw values).
    rows: query rows to evaluate (default: all); rows are independent.
    hybrid (causal only): dict with ``window`` (int >= 0), ``sel`` (selected
    key positions; entries outside [0, Sk) are ignored) and the
    full-precision rows ``q`` [Sq, D], ``k``, ``v`` [Sk, D]; see the module
    readings for which keys use them.
    Returns a dict with out [R, D], lse [R], m [R], l [R] and, on request,
    bound [R] (the float32 rounding envelope), weights [R, Sk] (the effective
    normalised attention weights) and tile_eps [R, n_tiles] (sum P_hat /
    sum P_tilde - 1 per visited tile, NaN where a tile was not visited).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    sq, d = q.shape
    sk = k.shape[0]
    if softmax_scale is None:
        softmax_scale = 1.0 / np.sqrt(d)
    if causal and sq != sk:
        raise ValueError("causal prefill requires Sq == Sk")
    assert kv_tile % mx.BLOCK == 0
    rows = np.arange(sq) if rows is None else np.asarray(rows, dtype=np.int64)
    r = rows.shape[0]
    if hybrid is not None:
        if not causal:
            raise ValueError("hybrid prefill is causal")
        win = int(hybrid["window"])
        assert win >= 0
        sel = np.asarray(hybrid.get("sel", []), dtype=np.int64).reshape(-1)
        in_sel = np.zeros(sk, dtype=bool)
        in_sel[sel[(sel >= 0) & (sel < sk)]] = True
        qf = np.asarray(hybrid["q"], dtype=np.float64)
        kf = np.asarray(hybrid["k"], dtype=np.float64)
        vf = np.asarray(hybrid["v"], dtype=np.float64)
    qr = q[rows]
    m = np.full(r, -np.inf)
    l = np.zeros(r)
    o = np.zeros((r, d))
    env = np.zeros(r)
    n_tiles = -(-sk // kv_tile)
    wts = np.zeros((r, sk)) if return_weights else None
    teps = np.full((r, n_tiles), np.nan) if return_tile_eps else None
    for j in range(n_tiles):
        t0, t1 = j * kv_tile, min((j + 1) * kv_tile, sk)
        n = t1 - t0
        keys = np.arange(t0, t1)
        visible = np.ones((r, n), dtype=bool)
        if causal:
            visible = keys[None, :] <= rows[:, None]
        if hybrid is not None:
            # Keys held in full precision for a row leave its 4-bit tiles.
            visible &= (keys[None, :] <= rows[:, None] - win) & ~in_sel[keys][None, :]
        act = visible.any(axis=1)
        if not act.any():
            continue
        ia = np.nonzero(act)[0]
        vis = visible[ia]
        s = softmax_scale * (qr[ia] @ k[t0:t1].T)
        s_vis = np.where(vis, s, -np.inf)
        m_old = m[ia]
        m_new = np.maximum(m_old, s_vis.max(axis=1))
        alpha = np.where(np.isfinite(m_old), np.exp(m_old - m_new), 0.0)
        pt = np.where(vis, np.exp(np.where(vis, s, 0.0) - m_new[:, None]), 0.0)
        if _perturb is not None:
            pt = _perturb(pt, s, m_new)
        npad = -(-n // mx.BLOCK) * mx.BLOCK
        ptp = np.zeros((ia.shape[0], npad))
        ptp[:, :n] = pt
        if quantize_p:
            php, e = _quantize_p_rows(ptp, p_rule, p_qmax)
            ph = php[:, :n]
        else:
            ph, e = pt, None
        add_l = ph.sum(axis=1) if l_from_quantized else pt.sum(axis=1)
        l[ia] = alpha * l[ia] + add_l
        o[ia] = alpha[:, None] * o[ia] + ph @ v[t0:t1]
        m[ia] = m_new
        if envelope and quantize_p:
            sp = np.zeros_like(ptp)
            sp[:, :n] = np.where(vis, s, 0.0)
            env[ia] = alpha * env[ia] + _envelope_tile(ptp, php, e, sp, m_new, p_rule, p_qmax)
        elif envelope:
            env[ia] = alpha * env[ia]
        if return_weights:
            wts[ia] *= alpha[:, None]
            wts[ia, t0:t1] = ph
        if return_tile_eps:
            with np.errstate(invalid="ignore", divide="ignore"):
                teps[ia, j] = ph.sum(axis=1) / pt.sum(axis=1) - 1.0
    if hybrid is not None:
        # One update with every full-precision key of each row, P unquantised.
        keys = np.arange(sk)
        hv = (keys[None, :] <= rows[:, None]) & ((keys[None, :] > rows[:, None] - win) | in_sel[None, :])
        ia = np.nonzero(hv.any(axis=1))[0]
        if ia.size:
            vis = hv[ia]
            s = softmax_scale * (qf[rows[ia]] @ kf.T)
            m_old = m[ia]
            m_new = np.maximum(m_old, np.where(vis, s, -np.inf).max(axis=1))
            alpha = np.where(np.isfinite(m_old), np.exp(m_old - m_new), 0.0)
            p = np.where(vis, np.exp(np.where(vis, s, 0.0) - m_new[:, None]), 0.0)
            l[ia] = alpha * l[ia] + p.sum(axis=1)
            o[ia] = alpha[:, None] * o[ia] + p @ vf
            m[ia] = m_new
            env[ia] = alpha * env[ia]
            if return_weights:
                wts[ia] = wts[ia] * alpha[:, None] + p
    with np.errstate(invalid="ignore", divide="ignore"):
        out = o / l[:, None]
        lse = m + np.log(l)
    res = {"out": out, "lse": lse, "m": m, "l": l}
    if envelope:
        vmax = np.abs(v).max() if v.size else 0.0
        denom = l - env
        with np.errstate(invalid="ignore", divide="ignore"):
            res["bound"] = np.where(env == 0, 0.0,
                                    np.where(denom > 0, env * 2.0 * vmax / denom, np.inf))
    if return_weights:
        with np.errstate(invalid="ignore", divide="ignore"):
            res["weights"] = wts / l[:, None]
    if return_tile_eps:
        res["tile_eps"] = teps
    return res


def prefill(q, k, v, **kw):
    """Multi-head prefill: q [B, Hq, Sq, D], k/v [B, Hkv, Sk, D] (float64).

    Query head g reads KV head g // (Hq / Hkv) (grouped-query attention).
    Keyword arguments are those of :func:`prefill_head`; ``rows`` may be a
    dict {(b, hq): row indices} to evaluate a sample of rows per head.
    Returns (out [B, Hq, R, D], lse [B, Hq, R], bound or None).
    """
    bsz, hq, sq, d = q.shape
    hkv = k.shape[1]
    assert hq % hkv == 0
    g = hq // hkv
    rows = kw.pop("rows", None)
    outs, lses, bnds = [], [], []
    for b in range(bsz):
        ob, lb, bb = [], [], []
        for h in range(hq):
            rr = rows[(b, h)] if isinstance(rows, dict) else rows
            res = prefill_head(q[b, h], k[b, h // g], v[b, h // g], rows=rr, **kw)
            ob.append(res["out"])
            lb.append(res["lse"])
            bb.append(res.get("bound"))
        outs.append(np.stack(ob))
        lses.append(np.stack(lb))
        bnds.append(bb)
    bound = None
    if kw.get("envelope"):
        bound = np.stack([np.stack(x) for x in bnds])
    return np.stack(outs), np.stack(lses), bound


def decode_head(q_hat, k_hat, v_hat, ctx, softmax_scale=None, *, hybrid=None):
    """Single-query softmax attention over the first ``ctx`` cache tokens.

    q_hat: [D] dequantised MXFP4 query; k_hat, v_hat: [>= ctx, D] dequantised
    MXFP4 cache rows.  ``hybrid`` (optional) is a dict with
      tokens: int array of token positions held in bf16 (window and selected),
      q: [D] bf16 query values, k, v: [len(tokens), D] bf16 rows.
    Those tokens use q . k in bf16 values; every other token t < ctx uses the
    4-bit operands.  One softmax covers the union (each token once), in
    float64; P is not quantised.  Returns (out [D], lse).
    """
    d = q_hat.shape[0]
    if softmax_scale is None:
        softmax_scale = 1.0 / np.sqrt(d)
    k_hat = np.asarray(k_hat, dtype=np.float64)[:ctx]
    v_hat = np.asarray(v_hat, dtype=np.float64)[:ctx]
    s = softmax_scale * (k_hat @ np.asarray(q_hat, dtype=np.float64))
    vals = v_hat.copy()
    if hybrid is not None:
        toks = np.asarray(hybrid["tokens"], dtype=np.int64)
        assert np.unique(toks).shape[0] == toks.shape[0], "a token may be held once"
        assert ((toks >= 0) & (toks < ctx)).all()
        s[toks] = softmax_scale * (np.asarray(hybrid["k"], np.float64) @ np.asarray(hybrid["q"], np.float64))
        vals[toks] = np.asarray(hybrid["v"], dtype=np.float64)
    mx_ = s.max()
    p = np.exp(s - mx_)
    den = p.sum()
    return (p @ vals) / den, mx_ + np.log(den)


def decode(q_hat, k_hat, v_hat, ctx_len, softmax_scale=None, pairs=None, hybrid=None):
    """Multi-head decode: q_hat [B, Hq, D], caches [B, Hkv, T, D].

    ``pairs`` selects (b, hq) pairs to evaluate (default: all);
    ``hybrid`` maps (b, hkv) -> dict(tokens, k, v) with ``q_bf16`` [B, Hq, D]
    under key "q".  Returns dict {(b, hq): (out [D], lse)}.
    """
    bsz, hq, d = q_hat.shape
    hkv = k_hat.shape[1]
    g = hq // hkv
    if pairs is None:
        pairs = [(b, h) for b in range(bsz) for h in range(hq)]
    res = {}
    for (b, h) in pairs:
        hy = None
        if hybrid is not None:
            ent = hybrid["sets"][(b, h // g)]
            hy = {"tokens": ent["tokens"], "k": ent["k"], "v": ent["v"],
                  "q": hybrid["q"][b, h]}
        res[(b, h)] = decode_head(q_hat[b, h], k_hat[b, h // g], v_hat[b, h // g],
                                  int(ctx_len[b]), softmax_scale, hybrid=hy)
    return res
