"""Pins for the oracle's prefill and decode (CPU only).

The oracle is checked against textbook softmax attention (quantisation off),
a direct whole-row PNQ computation (tile wider than the sequence), the
normalisation invariant PNQ guarantees, the output-neutrality of Smooth-QK,
and the limits of hybrid decode and prefill (with a closed-form key count for
the window and the selected set).  A planted float32-sized perturbation of
the exponentials checks that the rounding envelope covers what it claims.
"""

import numpy as np
import pytest

from oracle import attention, mx, smooth


def _textbook(q, k, v, causal, scale):
    """softmax(scale * q k^T) v written out directly, in float64."""
    s = scale * (q @ k.T)
    if causal:
        s = np.where(np.tril(np.ones_like(s, dtype=bool)), s, -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    return (p / p.sum(axis=1, keepdims=True)) @ v


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kv_tile", [32, 64, 128, 256])
@pytest.mark.parametrize("seq", [1, 77, 200, 320])
def test_quantisation_off_equals_textbook(causal, kv_tile, seq):
    q, k, v = _rand((seq, 64), 1), _rand((seq, 64), 2), _rand((seq, 64), 3)
    sc = 1 / np.sqrt(64)
    res = attention.prefill_head(q, k, v, causal=causal, kv_tile=kv_tile, quantize_p=False)
    np.testing.assert_allclose(res["out"], _textbook(q, k, v, causal, sc), rtol=0, atol=1e-12)


def test_non_causal_rectangular_and_row_subset():
    q, k, v = _rand((40, 128), 4), _rand((300, 128), 5), _rand((300, 128), 6)
    sc = 0.1
    res = attention.prefill_head(q, k, v, softmax_scale=sc, kv_tile=64, quantize_p=False,
                                 rows=[0, 7, 39])
    np.testing.assert_allclose(res["out"], _textbook(q, k, v, False, sc)[[0, 7, 39]], atol=1e-12)


def _direct_pnq(q, k, v, causal, scale, rule, qmax):
    """Whole-row PNQ: exponentials against the row maximum, quantised in
    32-key blocks from key 0, normaliser from the quantised values."""
    sq, sk = q.shape[0], k.shape[0]
    out = np.zeros((sq, v.shape[1]))
    for i in range(sq):
        s = scale * (k @ q[i])
        vis = np.ones(sk, dtype=bool) if not causal else np.arange(sk) <= i
        mrow = s[vis].max()
        pt = np.where(vis, np.exp(np.where(vis, s, 0) - mrow), 0.0)
        npad = -(-sk // 32) * 32
        ptp = np.zeros(npad)
        ptp[:sk] = pt
        codes, sb = mx.quantize_blocks(ptp[None], rule, qmax)
        ph = mx.dequantize_blocks(codes, sb)[0, :sk]
        out[i] = ph @ v / ph.sum()
    return out


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("rule", [mx.RULE_OCP, mx.RULE_UOS])
def test_single_tile_equals_direct_whole_row(causal, rule):
    q, k, v = _rand((96, 64), 7), _rand((96, 64), 8), _rand((96, 64), 9)
    sc = 1 / 8
    res = attention.prefill_head(q, k, v, causal=causal, kv_tile=128, p_rule=rule)
    np.testing.assert_allclose(res["out"], _direct_pnq(q, k, v, causal, sc, rule, 7.25),
                               atol=1e-12)


@pytest.mark.parametrize("kv_tile", [32, 128])
def test_pnq_weights_normalised(kv_tile):
    q, k, v = _rand((130, 64), 10) * 2, _rand((130, 64), 11), _rand((130, 64), 12)
    res = attention.prefill_head(q, k, v, causal=True, kv_tile=kv_tile, return_weights=True)
    w = res["weights"]
    assert (w >= 0).all()
    np.testing.assert_allclose(w.sum(axis=1), 1.0, atol=1e-12)
    np.testing.assert_allclose(res["out"], w @ v, atol=1e-12)
    # The tile that sets the maximum holds an exponential equal to 1, which
    # both scale rules code exactly, so l >= 1.
    assert (res["l"] >= 1.0 - 1e-15).all()
    # Causal: weights above the diagonal are exactly zero.
    assert (np.triu(w, 1) == 0).all()
    # Every output channel lies inside the range of the values.
    assert (np.abs(res["out"]) <= np.abs(v).max(axis=0) + 1e-12).all()


def test_baseline_normaliser_differs_and_matches_direct():
    q, k, v = _rand((64, 64), 13) * 2, _rand((64, 64), 14), _rand((64, 64), 15)
    base = attention.prefill_head(q, k, v, kv_tile=64, l_from_quantized=False, return_weights=True)
    pnq = attention.prefill_head(q, k, v, kv_tile=64)
    # Baseline: the weights of a row sum to sum(P_hat)/sum(P_tilde), not 1.
    s = (q @ k.T) / 8
    pt = np.exp(s - s.max(axis=1, keepdims=True))
    codes, sb = mx.quantize_blocks(pt)
    ph = mx.dequantize_blocks(codes, sb)
    np.testing.assert_allclose(base["weights"].sum(axis=1), ph.sum(1) / pt.sum(1), atol=1e-12)
    np.testing.assert_allclose(base["out"], (ph @ v) / pt.sum(1)[:, None], atol=1e-12)
    assert np.abs(base["out"] - pnq["out"]).max() > 1e-6


def test_tile_width_changes_pnq_but_not_exact_attention():
    q, k, v = _rand((256, 64), 16) * 2, _rand((256, 64), 17), _rand((256, 64), 18)
    a = attention.prefill_head(q, k, v, causal=True, kv_tile=32)["out"]
    b = attention.prefill_head(q, k, v, causal=True, kv_tile=256)["out"]
    assert np.abs(a - b).max() > 1e-6
    a0 = attention.prefill_head(q, k, v, causal=True, kv_tile=32, quantize_p=False)["out"]
    b0 = attention.prefill_head(q, k, v, causal=True, kv_tile=256, quantize_p=False)["out"]
    np.testing.assert_allclose(a0, b0, atol=1e-12)


def test_tile_mass_loss_diagnostic():
    """The per-tile mass change sum(P_hat)/sum(P_tilde) - 1 is defined on every
    visited tile and is small; this is reported, not a pass/fail target."""
    q, k, v = _rand((256, 128), 19), _rand((256, 128), 20), _rand((256, 128), 21)
    res = attention.prefill_head(q, k, v, causal=True, kv_tile=128, return_tile_eps=True)
    eps = res["tile_eps"]
    assert np.isnan(eps[:128, 1]).all() and np.isfinite(eps[128:, 1]).all()
    assert np.nanmax(np.abs(eps)) < 0.5


def test_smoothing_is_output_neutral_without_quantisation():
    rng = np.random.default_rng(22)
    qb = rng.standard_normal((2, 64, 64)).astype(np.float32)   # [Hq, S, D]
    kb = rng.standard_normal((1, 64, 64)).astype(np.float32)
    kb[:, :, 5] *= 12
    v = rng.standard_normal((64, 64))
    qs, ks = smooth.calibrate(qb, kb)
    q_sm = smooth.apply(qb, qs).astype(np.float64)
    k_sm = smooth.apply(kb, ks).astype(np.float64)
    for h in range(2):
        a = attention.prefill_head(qb[h].astype(np.float64), kb[0].astype(np.float64), v,
                                   quantize_p=False)["out"]
        b = attention.prefill_head(q_sm[h], k_sm[0], v, quantize_p=False)["out"]
        np.testing.assert_allclose(a, b, atol=2e-6)
    # With power-of-two factors the float32 rescale is exact, so the smoothed
    # logits, and the output, are identical.
    p2 = np.exp2(np.round(np.log2(qs.astype(np.float64)))).astype(np.float32)
    qp = smooth.apply(qb, p2).astype(np.float64)
    kp = smooth.apply(kb, (1.0 / p2[:1]).astype(np.float32)).astype(np.float64)
    np.testing.assert_array_equal(qp @ kp[0].T, qb.astype(np.float64) @ kb[0].astype(np.float64).T)


def test_envelope_covers_planted_float32_errors():
    """Exponentials perturbed by relative errors inside the envelope model
    (as a float32 implementation would) move each output by at most the
    reported bound (plus the 2e-3 slack used on the GPU this is far under)."""
    rng = np.random.default_rng(23)
    q, k, v = rng.standard_normal((256, 64)) * 2, rng.standard_normal((256, 64)), rng.standard_normal((256, 64))
    qc, qs = mx.quantize(q, axis=1)
    kc, ks = mx.quantize(k, axis=1)
    vc, vs = mx.quantize(v, axis=0)
    qh, kh, vh = mx.dequantize(qc, qs, 1), mx.dequantize(kc, ks, 1), mx.dequantize(vc, vs, 0)
    for rule in (mx.RULE_OCP, mx.RULE_UOS):
        ref = attention.prefill_head(qh, kh, vh, causal=True, p_rule=rule, envelope=True)
        for trial in range(3):
            noise_rng = np.random.default_rng(100 + trial)

            def perturb(pt, s, m_new):
                eta = attention.ETA0 + attention.ETA1 * (np.abs(s) + np.abs(m_new)[:, None])
                f = 1 + noise_rng.uniform(-1, 1, size=pt.shape) * eta
                return np.where(pt == 1.0, 1.0, pt * f)

            got = attention.prefill_head(qh, kh, vh, causal=True, p_rule=rule, _perturb=perturb)
            diff = np.abs(got["out"] - ref["out"]).max(axis=1)
            assert (diff <= ref["bound"] + 1e-12).all()


def test_decode_equals_prefill_single_row():
    rng = np.random.default_rng(24)
    k, v = rng.standard_normal((500, 128)), rng.standard_normal((500, 128))
    q = rng.standard_normal(128)
    out, lse = attention.decode_head(q, k, v, 437)
    ref = attention.prefill_head(q[None], k[:437], v[:437], kv_tile=64, quantize_p=False)
    np.testing.assert_allclose(out, ref["out"][0], atol=1e-12)
    np.testing.assert_allclose(lse, ref["lse"][0], atol=1e-12)


def test_hybrid_decode_limits():
    rng = np.random.default_rng(25)
    ctx, d = 300, 64
    kb, vb, qb = rng.standard_normal((ctx, d)), rng.standard_normal((ctx, d)), rng.standard_normal(d)
    kc, ks = mx.quantize(kb, axis=1)
    vc, vs = mx.quantize(vb, axis=1)
    qc, qs = mx.quantize(qb[None], axis=1)
    kh, vh, qh = mx.dequantize(kc, ks, 1), mx.dequantize(vc, vs, 1), mx.dequantize(qc, qs, 1)[0]
    fp4 = attention.decode_head(qh, kh, vh, ctx)
    none = attention.decode_head(qh, kh, vh, ctx, hybrid={"tokens": np.zeros(0, int),
                                                           "q": qb, "k": np.zeros((0, d)),
                                                           "v": np.zeros((0, d))})
    np.testing.assert_allclose(none[0], fp4[0], atol=1e-15)
    allbf = attention.decode_head(qh, kh, vh, ctx, hybrid={"tokens": np.arange(ctx), "q": qb,
                                                           "k": kb, "v": vb})
    np.testing.assert_allclose(allbf[0], _textbook(qb[None], kb, vb, False, 1 / 8)[0], atol=1e-12)
    # A partial set: the result is the softmax over the token-wise mixture.
    toks = np.array([3, 100, 250, 299])
    mix_k, mix_v = kh.copy(), vh.copy()
    mix_k[toks], mix_v[toks] = kb[toks], vb[toks]
    s = (mix_k @ qh) / 8
    s[toks] = (kb[toks] @ qb) / 8
    p = np.exp(s - s.max())
    part = attention.decode_head(qh, kh, vh, ctx, hybrid={"tokens": toks, "q": qb,
                                                          "k": kb[toks], "v": vb[toks]})
    np.testing.assert_allclose(part[0], (p @ mix_v) / p.sum(), atol=1e-12)
    with pytest.raises(AssertionError):
        attention.decode_head(qh, kh, vh, ctx, hybrid={"tokens": np.array([3, 3]), "q": qb,
                                                       "k": kb[:2], "v": vb[:2]})


@pytest.mark.parametrize("rule", [mx.RULE_OCP, mx.RULE_UOS])
def test_envelope_flags_and_covers_midpoints_and_scale_boundaries(rule):
    """Logits placed within the envelope of E2M1 midpoints and of a scale
    boundary: the oracle must flag them, and flipping them (as a float32
    implementation may) must stay inside the reported bound."""
    d, n = 64, 96
    rng = np.random.default_rng(31)
    q = np.zeros((1, d)); q[0, 0] = 1.0
    k = np.zeros((n, d))
    v = rng.standard_normal((n, d))
    tiny = 1e-9
    p = np.full(n, np.exp(-30.0))
    # Block 0 holds the maximum (P = 1, scale 2^-2 under both rules) and
    # exponentials sitting on the midpoints below 4 in scale units.
    p[0] = 1.0
    p[1:7] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5]) * 2.0 ** -2 * (1 + tiny)
    # Block 1: maximum 6 * 2^-5 (scale 2^-5 under both rules) and the last
    # midpoint, 5.
    p[32] = 6 * 2.0 ** -5
    p[33] = 5 * 2.0 ** -5 * (1 - tiny)
    # Block 2: maximum a hair below a scale boundary of the rule.
    bnd = 2.0 ** -3 if rule == mx.RULE_OCP else 7.25 * 2.0 ** -6
    p[64] = bnd * (1 - tiny)
    p[65:72] = bnd * np.linspace(0.3, 0.9, 7)
    k[:, 0] = np.log(p)
    ref = attention.prefill_head(q, k, v, softmax_scale=1.0, kv_tile=128, p_rule=rule,
                                 envelope=True)
    assert ref["bound"][0] > 0

    def scaled(f):
        return lambda pt, s, m_new: np.where(pt == 1.0, 1.0, pt * f)

    moved = 0.0
    for f in (1 + 3 * tiny, 1 - 3 * tiny):
        got = attention.prefill_head(q, k, v, softmax_scale=1.0, kv_tile=128, p_rule=rule,
                                     _perturb=scaled(f))
        diff = np.abs(got["out"] - ref["out"]).max()
        moved = max(moved, diff)
        assert diff <= ref["bound"][0] + 1e-12
    assert moved > 1e-4        # the planted flips really changed the result


# ---------------------------------------------------------------- hybrid prefill
def _hy(qf, kf, vf, window, sel):
    return {"window": window, "sel": np.asarray(sel, dtype=np.int64), "q": qf, "k": kf, "v": vf}


def test_hybrid_prefill_key_counts_closed_form():
    """All logits 0 (uniform weights) and a marker channel that is 1 only in
    the full-precision V rows: out[i, 0] = |full-precision keys of row i| /
    (i + 1), with i - W < t <= i the window and selected keys t <= i."""
    s, d, win, sel = 60, 32, 3, [2, 11, 40, 59]
    z = np.zeros((s, d))
    v4 = np.zeros((s, d))
    vf = np.zeros((s, d))
    vf[:, 0] = 1.0
    res = attention.prefill_head(z, z, v4, causal=True, kv_tile=32, quantize_p=False,
                                 hybrid=_hy(z, z, vf, win, sel))
    for i in range(s):
        n_win = min(win, i + 1)
        n_sel = sum(1 for t in sel if t <= i - win)
        assert res["out"][i, 0] == pytest.approx((n_win + n_sel) / (i + 1), abs=1e-14), i


def test_hybrid_prefill_limits():
    """Empty set and window 0: the 4-bit prefill, bit for bit.  Window >= Sq:
    textbook attention on the full-precision rows."""
    q, k, v = _rand((150, 64), 31) * 2, _rand((150, 64), 32), _rand((150, 64), 33)
    qf, kf, vf = _rand((150, 64), 34), _rand((150, 64), 35), _rand((150, 64), 36)
    plain = attention.prefill_head(q, k, v, causal=True, kv_tile=64)
    hyb0 = attention.prefill_head(q, k, v, causal=True, kv_tile=64, hybrid=_hy(qf, kf, vf, 0, []))
    assert np.array_equal(plain["out"], hyb0["out"]) and np.array_equal(plain["lse"], hyb0["lse"])
    allf = attention.prefill_head(q, k, v, causal=True, kv_tile=64, hybrid=_hy(qf, kf, vf, 150, [3, 77]))
    np.testing.assert_allclose(allf["out"], _textbook(qf, kf, vf, True, 1 / 8), atol=1e-12)


@pytest.mark.parametrize("kv_tile", [32, 64, 128])
@pytest.mark.parametrize("win, sel", [(0, [0, 5, 63, 64, 150]), (16, []), (40, [1, 2, 3, 100, 190]),
                                      (7, list(range(0, 200, 9)))])
def test_hybrid_prefill_quantisation_off_equals_textbook(kv_tile, win, sel):
    """With P unquantised and one operand set for both paths, splitting keys
    between the parts must leave textbook attention unchanged: a key counted
    twice or dropped fails."""
    q, k, v = _rand((200, 64), 37), _rand((200, 64), 38), _rand((200, 64), 39)
    res = attention.prefill_head(q, k, v, causal=True, kv_tile=kv_tile, quantize_p=False,
                                 hybrid=_hy(q, k, v, win, sel))
    np.testing.assert_allclose(res["out"], _textbook(q, k, v, True, 1 / 8), atol=1e-12)


def _direct_hybrid(q, k, v, qf, kf, vf, win, sel, scale, rule, qmax):
    """Whole-row hybrid PNQ written out per row: the 4-bit keys' exponentials
    against their own maximum, quantised in 32-key blocks from key 0, then
    the full-precision keys rescaled into the same softmax."""
    sq = q.shape[0]
    sel = set(sel)
    out = np.zeros((sq, v.shape[1]))
    for i in range(sq):
        f4 = [t for t in range(i + 1) if t <= i - win and t not in sel]
        hf = [t for t in range(i + 1) if t > i - win or t in sel]
        s4 = scale * (k[f4] @ q[i]) if f4 else np.zeros(0)
        sf = scale * (kf[hf] @ qf[i])
        m4 = s4.max() if f4 else -np.inf
        m = max(m4, sf.max())
        o = np.zeros(v.shape[1])
        l = 0.0
        if f4:
            row = np.zeros(-(-sq // 32) * 32)
            row[f4] = np.exp(s4 - m4)
            codes, sb = mx.quantize_blocks(row[None], rule, qmax)
            ph = mx.dequantize_blocks(codes, sb)[0, :sq]
            o += np.exp(m4 - m) * (ph @ v[:sq])
            l += np.exp(m4 - m) * ph.sum()
        pf = np.exp(sf - m)
        o += pf @ vf[hf]
        l += pf.sum()
        out[i] = o / l
    return out


@pytest.mark.parametrize("rule", [mx.RULE_OCP, mx.RULE_UOS])
def test_hybrid_prefill_single_tile_equals_direct(rule):
    q, k, v = _rand((96, 64), 40) * 2, _rand((96, 64), 41), _rand((96, 64), 42)
    qf, kf, vf = q + 0.1 * _rand((96, 64), 43), k + 0.1 * _rand((96, 64), 44), v + 0.1 * _rand((96, 64), 45)
    win, sel = 10, [0, 4, 30, 31, 70, 95]
    res = attention.prefill_head(q, k, v, causal=True, kv_tile=128, p_rule=rule,
                                 hybrid=_hy(qf, kf, vf, win, sel))
    np.testing.assert_allclose(res["out"], _direct_hybrid(q, k, v, qf, kf, vf, win, sel, 1 / 8, rule, 7.25),
                               atol=1e-12)


def test_hybrid_prefill_weights_normalised():
    q, k, v = _rand((130, 64), 46) * 2, _rand((130, 64), 47), _rand((130, 64), 48)
    res = attention.prefill_head(q, k, v, causal=True, kv_tile=32, return_weights=True,
                                 hybrid=_hy(q * 1.01, k, v, 20, [5, 6, 64, 100]))
    w = res["weights"]
    assert (w >= 0).all()
    np.testing.assert_allclose(w.sum(axis=1), 1.0, atol=1e-12)
    assert np.all(np.triu(w, 1) == 0)


# ---------------------------------------------------------------- two-tile golden
def _golden_rows(name):
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", name)
    with open(path) as f:
        return [ln.split() for ln in (l.strip() for l in f) if ln and not ln.startswith("#")]


def _two_tile_case(case):
    """The inputs of tests/golden/two_tile_running_max.txt (see its header)."""
    if case in ("A", "B"):
        logit = np.zeros(34)
        logit[32] = np.log(0.3 if case == "A" else 0.46875)
        logit[33] = np.log(0.2)
        ia, ib = 32, 33
    else:
        logit = np.full(64, -60.0)
        logit[0], logit[1] = np.log(0.3), np.log(0.2)
        logit[32:] = 0.0
        ia, ib = 0, 1
    k = np.stack([logit, np.zeros_like(logit)], axis=1)
    v = np.zeros_like(k)
    v[ia, 0] = 1.0
    v[ib, 1] = 1.0
    return np.array([[1.0, 0.0]]), k, v


@pytest.mark.parametrize("row", _golden_rows("two_tile_running_max.txt"), ids=" ".join)
def test_two_tile_running_max_golden(row):
    """Hand-worked two-tile rows: the exponentials of a tile are quantised
    against the running maximum after that tile (not the tile's own maximum,
    not the row's final one), earlier tiles are rescaled, and l follows the
    chosen rule (HiFA4, Abstract; MXAttention, Abstract)."""
    case, rule, lmode = row[:3]
    w_a, w_b, lval = (float(x) for x in row[3:])
    q, k, v = _two_tile_case(case)
    res = attention.prefill_head(q, k, v, softmax_scale=1.0, kv_tile=32,
                                 p_rule=mx.RULE_OCP if rule == "ocp" else mx.RULE_UOS,
                                 l_from_quantized=(lmode == "pnq"))
    np.testing.assert_allclose(res["l"], [lval], rtol=0, atol=1e-12)
    np.testing.assert_allclose(res["out"][0], [w_a / lval, w_b / lval], rtol=0, atol=1e-12)
    np.testing.assert_allclose(res["lse"], [np.log(lval)], rtol=0, atol=1e-12)
    np.testing.assert_allclose(res["m"], [0.0], atol=0)


# ---------------------------------------------------------------- GQA wrappers
def _gqa_inputs(seed, b=2, hq=6, hkv=2, s=70, d=64):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((b, hq, s, d)), rng.standard_normal((b, hkv, s, d)),
            rng.standard_normal((b, hkv, s, d)))


@pytest.mark.parametrize("causal", [False, True])
def test_multihead_prefill_gqa_equals_repeated_kv(causal):
    """attention.prefill maps query head g to a KV head; checked against the
    repeat-each-KV-head-consecutively form of grouped-query attention
    (np.repeat along the head axis), with textbook softmax when P is not
    quantised and the direct whole-row PNQ when one tile spans the row."""
    q, k, v = _gqa_inputs(21)
    g = q.shape[1] // k.shape[1]
    kr, vr = np.repeat(k, g, axis=1), np.repeat(v, g, axis=1)
    sc = 1 / 8
    out0, lse0, _ = attention.prefill(q, k, v, causal=causal, quantize_p=False)
    out1, _, bnd = attention.prefill(q, k, v, causal=causal, kv_tile=128, envelope=True)
    assert out0.shape == q.shape and lse0.shape == q.shape[:3] and bnd.shape == q.shape[:3]
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            np.testing.assert_allclose(out0[b, h], _textbook(q[b, h], kr[b, h], vr[b, h], causal, sc), atol=1e-12)
            np.testing.assert_allclose(out1[b, h], _direct_pnq(q[b, h], kr[b, h], vr[b, h], causal, sc,
                                                               mx.RULE_OCP, 7.25), atol=1e-12)


def test_multihead_prefill_row_samples():
    q, k, v = _gqa_inputs(22)
    rows = {(b, h): np.array([0, 1 + h, 69 - b]) for b in range(2) for h in range(6)}
    full, _, _ = attention.prefill(q, k, v, causal=True)
    part, _, _ = attention.prefill(q, k, v, causal=True, rows=rows)
    for (b, h), r in rows.items():
        np.testing.assert_allclose(part[b, h], full[b, h, r], atol=0)


def test_multihead_decode_gqa_and_hybrid_sets():
    """attention.decode: each (b, hq) pair against textbook softmax over the
    KV head repeated per group; the hybrid sets, keyed by (b, KV head), are
    substituted into the repeated rows the same way."""
    rng = np.random.default_rng(23)
    b, hq, hkv, t, d = 2, 8, 2, 300, 64
    g = hq // hkv
    q = rng.standard_normal((b, hq, d))
    k, v = rng.standard_normal((b, hkv, t, d)), rng.standard_normal((b, hkv, t, d))
    ctx = np.array([300, 123])
    qb = q + 0.01 * rng.standard_normal(q.shape)
    sets = {}
    ks, vs = k.copy(), v.copy()
    for bb in range(b):
        for h in range(hkv):
            toks = np.sort(rng.choice(int(ctx[bb]), size=20, replace=False))
            kk, vv = rng.standard_normal((20, d)), rng.standard_normal((20, d))
            sets[(bb, h)] = {"tokens": toks, "k": kk, "v": vv}
            ks[bb, h, toks], vs[bb, h, toks] = kk, vv
    kr, vr = np.repeat(k, g, axis=1), np.repeat(v, g, axis=1)
    ksr, vsr = np.repeat(ks, g, axis=1), np.repeat(vs, g, axis=1)
    plain = attention.decode(q, k, v, ctx)
    pairs = [(0, 0), (0, 5), (1, 3), (1, 7)]
    hyb = attention.decode(q, k, v, ctx, pairs=pairs, hybrid={"sets": sets, "q": qb})
    assert sorted(plain) == [(bb, h) for bb in range(b) for h in range(hq)] and sorted(hyb) == sorted(pairs)
    sc = 1 / 8
    for (bb, h), (o, lse) in plain.items():
        c = int(ctx[bb])
        s = sc * (kr[bb, h, :c] @ q[bb, h])
        p = np.exp(s - s.max())
        np.testing.assert_allclose(o, p @ vr[bb, h, :c] / p.sum(), atol=1e-12)
        np.testing.assert_allclose(lse, s.max() + np.log(p.sum()), atol=1e-12)
    for (bb, h), (o, _) in hyb.items():
        c = int(ctx[bb])
        toks = sets[(bb, h // g)]["tokens"]
        s = sc * (kr[bb, h, :c] @ q[bb, h])
        s[toks] = sc * (ksr[bb, h, toks] @ qb[bb, h])
        vals = vr[bb, h, :c].copy()
        vals[toks] = vsr[bb, h, toks]
        p = np.exp(s - s.max())
        np.testing.assert_allclose(o, p @ vals / p.sum(), atol=1e-12)
