"""GPU parity of MXFP4 decode (plain and hybrid) and of vertical-line
selection against the oracle.  Decode outputs must match within 2e-3 max-abs
(P is not quantised, so no rounding envelope is involved); cache codes are
compared bit for bit; the top-k is compared exactly where the masses are
exact and, for float masses, on what is unique (indices clearly above or
below the threshold) with the rest checked for validity."""

import numpy as np
import pytest
import torch

import bit_microscaled_flashattention_amd as mxa
import synth
from oracle import attention, mx, rotate, select
from tests.helpers import (assert_codes_equal, check_selection, head_slice, host_f64, oracle_dequant,
                           oracle_quantize)

pytestmark = pytest.mark.gpu
DEV = "cuda"
ATOL = 2e-3


def _cache(k, v):
    return mxa.quantize(k, "hd"), mxa.quantize(v, "hd")


def _query(q):
    return mxa.quantize(q[:, :, None, :], "hd")


def _oracle_pair(q, k, v, ctx, pairs, hybrid_sets=None, q_bf=None):
    """Oracle decode on (b, hq) pairs from the generator tensors."""
    hq, hkv = q.shape[1], k.shape[1]
    g = hq // hkv
    res = {}
    qd_all = oracle_dequant(*oracle_quantize(host_f64(q[:, :, None, :]), "hd"), "hd")[:, :, 0]
    cache = {}
    for (b, h) in pairs:
        kv = h // g
        if (b, kv) not in cache:
            kk = host_f64(k[b:b + 1, kv:kv + 1])
            vv = host_f64(v[b:b + 1, kv:kv + 1])
            cache[(b, kv)] = (oracle_dequant(*oracle_quantize(kk, "hd"), "hd")[0, 0],
                              oracle_dequant(*oracle_quantize(vv, "hd"), "hd")[0, 0])
        kd, vd = cache[(b, kv)]
        hy = None
        if hybrid_sets is not None:
            toks, kr, vr = hybrid_sets[(b, kv)]
            hy = {"tokens": toks, "k": kr, "v": vr, "q": host_f64(q_bf[b, h])}
        res[(b, h)] = attention.decode_head(qd_all[b, h], kd, vd, int(ctx[b]), hybrid=hy)
    return res


def _compare(out, lse, ref, what):
    o = out.cpu().numpy()
    l = lse.cpu().numpy()
    worst = 0.0
    for (b, h), (ro, rl) in ref.items():
        err = np.abs(o[b, h] - ro).max()
        worst = max(worst, err)
        assert err <= ATOL, f"{what}: (b={b}, h={h}) err {err:.3e}"
        assert abs(l[b, h] - rl) <= 1e-3, f"{what}: lse (b={b}, h={h}) {l[b, h]} vs {rl}"
    print(f"  {what}: worst |err| {worst:.3e} over {len(ref)} pairs", flush=True)


@pytest.mark.parametrize("d, hq, hkv", [(128, 8, 2), (64, 4, 4), (128, 16, 2)])
def test_decode_small_ragged(d, hq, hkv):
    g = torch.Generator(device=DEV).manual_seed(31)
    b, tcap = 2, 1000
    q = torch.randn((b, hq, d), generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn((b, hkv, tcap, d), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((b, hkv, tcap, d), generator=g, device=DEV).to(torch.bfloat16)
    ctx = torch.tensor([1000, 577], dtype=torch.int32, device=DEV)
    print(f"decode small d={d} hq={hq} hkv={hkv}", flush=True)
    kc, vc = _cache(k, v)
    qh = _query(q)
    out, lse = mxa.decode(qh, kc, vc, ctx, split_len=256, return_lse=True)
    torch.cuda.synchronize()
    ref = _oracle_pair(q, k, v, ctx.cpu().numpy(), [(bb, h) for bb in range(b) for h in range(hq)])
    _compare(out, lse, ref, f"decode d={d} G={hq // hkv}")


def test_decode_split_and_tiny_context():
    g = torch.Generator(device=DEV).manual_seed(32)
    b, hq, hkv, tcap, d = 3, 4, 1, 700, 128
    q = torch.randn((b, hq, d), generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn((b, hkv, tcap, d), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((b, hkv, tcap, d), generator=g, device=DEV).to(torch.bfloat16)
    ctx = torch.tensor([1, 64, 700], dtype=torch.int32, device=DEV)
    kc, vc = _cache(k, v)
    qh = _query(q)
    outs = [mxa.decode(qh, kc, vc, ctx, split_len=s) for s in (64, 128, 2048)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert (o - outs[0]).abs().max().item() < 1e-5
    ref = _oracle_pair(q, k, v, ctx.cpu().numpy(), [(bb, h) for bb in range(b) for h in range(hq)])
    _compare(outs[0], mxa.decode(qh, kc, vc, ctx, split_len=64, return_lse=True)[1], ref, "split 64")
    # ctx = 1: the output is the first value row.
    vd = oracle_dequant(*oracle_quantize(host_f64(v[0:1, :, 0:1]), "hd"), "hd")[0, 0, 0]
    np.testing.assert_allclose(outs[0][0, 0].cpu().numpy(), vd, atol=1e-6)


def test_decode_dual_residual_query():
    """A dual-residual query (q1, q2) scores every 4-bit token with
    dequant(q1) + dequant(q2): parity with the oracle on that query, and the
    outputs move towards attention with the unquantised query."""
    g = torch.Generator(device=DEV).manual_seed(36)
    b, hq, hkv, tcap, d = 2, 8, 2, 1500, 128
    q = torch.randn((b, hq, d), generator=g, device=DEV).to(torch.bfloat16)
    q[:, :, 3] *= 12
    k = torch.randn((b, hkv, tcap, d), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((b, hkv, tcap, d), generator=g, device=DEV).to(torch.bfloat16)
    ctx = torch.tensor([1500, 999], dtype=torch.int32, device=DEV)
    kc, vc = _cache(k, v)
    q1, q2 = mxa.quantize_dual(q[:, :, None, :])
    print("decode dual-residual query", flush=True)
    out_d, lse_d = mxa.decode(q1, kc, vc, ctx, split_len=512, return_lse=True, q_res=q2)
    out_s = mxa.decode(q1, kc, vc, ctx, split_len=512)
    torch.cuda.synchronize()
    c1, s1, c2, s2 = mx.quantize_dual(host_f64(q[:, :, None, :]), axis=3)
    q_hat = (oracle_dequant(c1, s1, "hd") + oracle_dequant(c2, s2, "hd"))[:, :, 0]
    q_ex = host_f64(q)
    ref, ref_exact = {}, {}
    for bb in range(b):
        for h in range(hq):
            kv = h // (hq // hkv)
            kd = oracle_dequant(*oracle_quantize(host_f64(k[bb:bb + 1, kv:kv + 1]), "hd"), "hd")[0, 0]
            vd = oracle_dequant(*oracle_quantize(host_f64(v[bb:bb + 1, kv:kv + 1]), "hd"), "hd")[0, 0]
            ref[(bb, h)] = attention.decode_head(q_hat[bb, h], kd, vd, int(ctx[bb]))
            ref_exact[(bb, h)] = attention.decode_head(q_ex[bb, h], kd, vd, int(ctx[bb]))[0]
    _compare(out_d, lse_d, ref, "dual-residual decode")
    od, os_ = out_d.cpu().numpy(), out_s.cpu().numpy()
    err_d = np.mean([np.abs(od[bb, h] - ref_exact[(bb, h)]).mean() for (bb, h) in ref_exact])
    err_s = np.mean([np.abs(os_[bb, h] - ref_exact[(bb, h)]).mean() for (bb, h) in ref_exact])
    print(f"  mean |out - out(exact q)|: single {err_s:.3e}, dual {err_d:.3e}", flush=True)
    assert err_d < err_s / 2


def test_decode_hadamard_rotated_query_and_keys():
    """Query and K cache rotated by the Walsh-Hadamard transform before
    MXFP4 (V as is): cache codes bit-exact with the oracle's float32
    transform, decode parity on the rotated operands, and outputs closer to
    attention on the unquantised inputs than without the rotation when K
    has outlier channels."""
    g = torch.Generator(device=DEV).manual_seed(37)
    b, hq, hkv, tcap, d = 2, 8, 2, 1300, 128
    q = torch.randn((b, hq, d), generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn((b, hkv, tcap, d), generator=g, device=DEV)
    k[:, :, :, 7] *= 12
    k[:, :, :, 70] *= 12
    k = k.to(torch.bfloat16)
    v = torch.randn((b, hkv, tcap, d), generator=g, device=DEV).to(torch.bfloat16)
    ctx = torch.tensor([1300, 777], dtype=torch.int32, device=DEV)
    print("decode with rotated query and keys", flush=True)
    kc_r = mxa.quantize(k, "hd", hadamard=True)
    qh_r = mxa.quantize(q[:, :, None, :], "hd", hadamard=True)
    kc, vc = _cache(k, v)
    out_r, lse_r = mxa.decode(qh_r, kc_r, vc, ctx, split_len=512, return_lse=True)
    out_p = mxa.decode(_query(q), kc, vc, ctx, split_len=512)
    torch.cuda.synchronize()
    k_rot = rotate.hadamard_f32(host_f64(k).astype(np.float32), axis=3).astype(np.float64)
    q_rot = rotate.hadamard_f32(host_f64(q[:, :, None, :]).astype(np.float32), axis=3).astype(np.float64)
    kcodes, kscales = oracle_quantize(k_rot, "hd")
    assert_codes_equal(kc_r, kcodes, kscales, "rotated K cache")
    qd = oracle_dequant(*oracle_quantize(q_rot, "hd"), "hd")[:, :, 0]
    kd_all = oracle_dequant(kcodes, kscales, "hd")
    ref, ref_exact = {}, {}
    for bb in range(b):
        for h in range(hq):
            kv = h // (hq // hkv)
            vd = oracle_dequant(*oracle_quantize(host_f64(v[bb:bb + 1, kv:kv + 1]), "hd"), "hd")[0, 0]
            ref[(bb, h)] = attention.decode_head(qd[bb, h], kd_all[bb, kv], vd, int(ctx[bb]))
            ref_exact[(bb, h)] = attention.decode_head(host_f64(q[bb, h]), host_f64(k[bb, kv]),
                                                       host_f64(v[bb, kv]), int(ctx[bb]))[0]
    _compare(out_r, lse_r, ref, "rotated decode")
    orr, op = out_r.cpu().numpy(), out_p.cpu().numpy()
    err_r = np.mean([np.abs(orr[bb, h] - ref_exact[(bb, h)]).mean() for (bb, h) in ref_exact])
    err_p = np.mean([np.abs(op[bb, h] - ref_exact[(bb, h)]).mean() for (bb, h) in ref_exact])
    print(f"  mean |out - exact|: plain {err_p:.3e}, rotated {err_r:.3e}", flush=True)
    assert err_r < err_p


def _page_pool(c, page, ctx, seed, spare=7):
    """Scatter a contiguous MX cache [B, Hkv, T, D] into a shuffled pool of
    pages (plus `spare` pages of random bytes that nothing may read).  Pages
    wholly past a sequence's context get table entry -1."""
    b, hkv, t, d = c.shape
    maxp = t // page
    g = torch.Generator().manual_seed(seed)
    n_pages = b * maxp + spare
    perm = torch.randperm(n_pages, generator=g)[:b * maxp].reshape(b, maxp).to(torch.int32)
    used = (torch.arange(maxp)[None, :] * page) < ctx.cpu()[:, None].long()
    table = torch.where(used, perm, torch.full_like(perm, -1))
    if spare > 0:
        codes = torch.randint(0, 256, (n_pages, hkv, page, d // 2), generator=g, dtype=torch.uint8).to(DEV)
        scales = torch.randint(0, 256, (n_pages, hkv, page, d // 32), generator=g, dtype=torch.uint8).to(DEV)
    else:
        codes = torch.zeros((n_pages, hkv, page, d // 2), dtype=torch.uint8, device=DEV)
        scales = torch.zeros((n_pages, hkv, page, d // 32), dtype=torch.uint8, device=DEV)
    src_c = c.codes.reshape(b, hkv, maxp, page, d // 2).permute(0, 2, 1, 3, 4).reshape(b * maxp, hkv, page, d // 2)
    src_s = c.scales.reshape(b, hkv, maxp, page, d // 32).permute(0, 2, 1, 3, 4).reshape(b * maxp, hkv, page, d // 32)
    sel = used.reshape(-1).to(DEV)
    dst = perm.reshape(-1).long().to(DEV)[sel]
    codes[dst] = src_c[sel]
    scales[dst] = src_s[sel]
    pool = mxa.MX(codes, scales, (n_pages, hkv, page, d), "hd")
    return pool, table.contiguous().to(DEV)


@pytest.mark.parametrize("page, d, hq, hkv, split", [(32, 128, 8, 2, 1024), (64, 64, 4, 4, 512),
                                                     (256, 128, 16, 2, 2048), (128, 128, 8, 8, 8192)])
def test_decode_paged_matches_contiguous(page, d, hq, hkv, split):
    """The paged scan gives the contiguous scan's outputs bit for bit on the
    cache its pages spell out (shuffled pages, ragged contexts, pages past the
    context absent from the table), and the oracle's within tolerance."""
    g = torch.Generator(device=DEV).manual_seed(40 + page)
    b, tcap = 3, 2048
    q = torch.randn((b, hq, d), generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn((b, hkv, tcap, d), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((b, hkv, tcap, d), generator=g, device=DEV).to(torch.bfloat16)
    ctx = torch.tensor([2048, 1000, 33], dtype=torch.int32, device=DEV)
    kc, vc = _cache(k, v)
    kp, table = _page_pool(kc, page, ctx, seed=page)
    vp, _ = _page_pool(vc, page, ctx, seed=page)
    qh = _query(q)
    print(f"paged decode page={page} d={d} hq={hq} hkv={hkv} split={split}", flush=True)
    ref_o, ref_l = mxa.decode(qh, kc, vc, ctx, split_len=split, return_lse=True)
    got_o, got_l = mxa.decode_paged(qh, kp, vp, table, ctx, split_len=split, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(ref_o, got_o) and torch.equal(ref_l, got_l)
    pairs = [(0, 0), (1, hq - 1), (2, hq // 2)]
    _compare(got_o, got_l, _oracle_pair(q, k, v, ctx, pairs), f"paged page={page}")


def test_decode_paged_hybrid_and_dual_query():
    """A hybrid set and a dual-residual query over the paged cache: the same
    bits as over the contiguous cache."""
    g = torch.Generator(device=DEV).manual_seed(45)
    b, hq, hkv, tcap, d, page = 2, 8, 2, 4096, 128, 64
    q = torch.randn((b, hq, d), generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn((b, hkv, tcap, d), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((b, hkv, tcap, d), generator=g, device=DEV).to(torch.bfloat16)
    ctx = torch.tensor([4096, 2500], dtype=torch.int32, device=DEV)
    kc, vc = _cache(k, v)
    kp, table = _page_pool(kc, page, ctx, seed=3)
    vp, _ = _page_pool(vc, page, ctx, seed=3)
    hy, _ = _hybrid_inputs(q, k, v, ctx, 64, 50, 64, seed=9)
    q1, q2 = mxa.quantize_dual(q[:, :, None, :])
    print("paged decode with hybrid set and dual query", flush=True)
    ref = mxa.decode(q1, kc, vc, ctx, split_len=2048, hybrid=hy, q_bf16=q.contiguous(), q_res=q2)
    got = mxa.decode_paged(q1, kp, vp, table, ctx, split_len=2048, hybrid=hy, q_bf16=q.contiguous(), q_res=q2)
    torch.cuda.synchronize()
    assert torch.equal(ref, got)


@pytest.mark.parametrize("d,hq,hkv", [(128, 32, 8), (64, 8, 8), (128, 16, 2)])
def test_decode_encodes_bf16_query_in_scan(d, hq, hkv):
    """A bf16 query handed to the scan unencoded gives the bits of the same
    decode on the quantiser's codes: plain, hybrid and paged scans.  Queries
    carry outlier channels and tiny blocks so several scale bytes, including
    the integer encoder's range, occur."""
    g = torch.Generator(device=DEV).manual_seed(46)
    b, tcap, page = 3, 4096, 64
    qf = torch.randn((b, hq, d), generator=g, device=DEV)
    qf[:, :, 5] *= 40
    qf[0, 0, :32] *= 1e-38
    q = qf.to(torch.bfloat16)
    k = torch.randn((b, hkv, tcap, d), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((b, hkv, tcap, d), generator=g, device=DEV).to(torch.bfloat16)
    ctx = torch.tensor([4096, 1777, 40], dtype=torch.int32, device=DEV)
    kc, vc = _cache(k, v)
    qh = mxa.quantize(q[:, :, None, :], "hd")
    print(f"decode with the query encoded in the scan d={d} hq={hq} hkv={hkv}", flush=True)
    ref_o, ref_l = mxa.decode(qh, kc, vc, ctx, split_len=1024, return_lse=True)
    got_o, got_l = mxa.decode(q, kc, vc, ctx, split_len=1024, return_lse=True)
    hy, _ = _hybrid_inputs(q, k, v, ctx, 64, 50, 64, seed=11)
    ref_h = mxa.decode(qh, kc, vc, ctx, split_len=1024, hybrid=hy, q_bf16=q.contiguous())
    got_h = mxa.decode(q, kc, vc, ctx, split_len=1024, hybrid=hy)
    kp, table = _page_pool(kc, page, ctx, seed=5)
    vp, _ = _page_pool(vc, page, ctx, seed=5)
    got_p = mxa.decode_paged(q[:, :, None, :], kp, vp, table, ctx, split_len=1024)
    torch.cuda.synchronize()
    assert torch.equal(ref_o, got_o) and torch.equal(ref_l, got_l)
    assert torch.equal(ref_h, got_h)
    assert torch.equal(ref_o, got_p)


def _hybrid_inputs(q, k, v, ctx, window, n_sel, max_sel, seed):
    """Seeded selected sets (ascending, below ctx-window) and the gathered
    bf16 rows the decode reads."""
    rng = np.random.default_rng(seed)
    b, hkv, tcap, d = k.shape
    idx = np.full((b, hkv, max_sel), -1, dtype=np.int32)
    nsel = np.zeros((b, hkv), dtype=np.int32)
    sets = {}
    kh, vh = host_f64(k), host_f64(v)
    for bb in range(b):
        c = int(ctx[bb])
        lim = max(c - window, 0)
        for h in range(hkv):
            n = min(n_sel, lim)
            sel = np.sort(rng.choice(lim, size=n, replace=False)) if n > 0 else np.zeros(0, np.int64)
            idx[bb, h, :n] = sel
            nsel[bb, h] = n
            win = np.arange(max(c - window, 0), c)
            toks = np.concatenate([sel, win]).astype(np.int64)
            sets[(bb, h)] = (toks, kh[bb, h, toks], vh[bb, h, toks])
    idx_t = torch.from_numpy(idx).to(DEV)
    gidx = idx_t.clamp_min(0).long()
    k_sel = torch.gather(k, 2, gidx[..., None].expand(-1, -1, -1, d)).contiguous()
    v_sel = torch.gather(v, 2, gidx[..., None].expand(-1, -1, -1, d)).contiguous()
    # Window rows: row w is token ctx - window + w (rows before token 0 unused).
    k_win = torch.zeros((b, hkv, window, d), dtype=k.dtype, device=DEV)
    v_win = torch.zeros_like(k_win)
    for bb in range(b):
        c = int(ctx[bb])
        lo = max(c - window, 0)
        k_win[bb, :, window - (c - lo):] = k[bb, :, lo:c]
        v_win[bb, :, window - (c - lo):] = v[bb, :, lo:c]
    hy = {"idx": idx_t, "n_sel": torch.from_numpy(nsel).to(DEV), "k_sel": k_sel, "v_sel": v_sel,
          "k_win": k_win, "v_win": v_win, "window": window}
    return hy, sets


@pytest.mark.parametrize("window, n_sel", [(64, 40), (0, 0), (0, 30), (50, 0), (880, 10)])
def test_hybrid_decode_small(window, n_sel):
    g = torch.Generator(device=DEV).manual_seed(33)
    b, hq, hkv, tcap, d = 2, 8, 2, 900, 128
    q = torch.randn((b, hq, d), generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn((b, hkv, tcap, d), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((b, hkv, tcap, d), generator=g, device=DEV).to(torch.bfloat16)
    ctx = torch.tensor([900, 611], dtype=torch.int32, device=DEV)
    print(f"hybrid small window={window} n_sel={n_sel}", flush=True)
    kc, vc = _cache(k, v)
    qh = _query(q)
    max_sel = max(n_sel, 1) + 8
    window_arg = min(window, tcap)
    hy, sets = _hybrid_inputs(q, k, v, ctx.cpu().numpy(), window_arg, n_sel, max_sel, 7)
    out, lse = mxa.decode(qh, kc, vc, ctx, split_len=128, hybrid=hy, q_bf16=q.contiguous(), return_lse=True)
    torch.cuda.synchronize()
    pairs = [(bb, h) for bb in range(b) for h in range(hq)]
    ref = _oracle_pair(q, k, v, ctx.cpu().numpy(), pairs, hybrid_sets=sets, q_bf=q)
    _compare(out, lse, ref, f"hybrid W={window} n={n_sel}")
    if window == 0 and n_sel == 0:
        plain = mxa.decode(qh, kc, vc, ctx, split_len=128)
        torch.cuda.synchronize()
        assert (plain - out).abs().max().item() < 1e-5


def test_decode_at_the_slot_limit():
    """The largest number of partial slots a call accepts (4096 per sequence:
    a 262144-token cache in splits of 64) against the oracle, with a ragged
    context that leaves the last 13 tokens out; one slot more is refused
    before launch."""
    g = torch.Generator(device=DEV).manual_seed(36)
    b, hq, hkv, tcap, d, split = 1, 4, 1, 4096 * 64, 64, 64
    q = torch.randn((b, hq, d), generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn((b, hkv, tcap, d), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((b, hkv, tcap, d), generator=g, device=DEV).to(torch.bfloat16)
    ctx = torch.tensor([tcap - 13], dtype=torch.int32, device=DEV)
    print("decode: 4096 slots of 64 tokens", flush=True)
    kc, vc = _cache(k, v)
    out, lse = mxa.decode(_query(q), kc, vc, ctx, split_len=split, return_lse=True)
    torch.cuda.synchronize()
    ref = _oracle_pair(q, k, v, ctx.cpu().numpy(), [(0, h) for h in range(hq)])
    _compare(out, lse, ref, "4096 slots")
    k2 = torch.zeros((b, hkv, tcap + 64, d), dtype=torch.bfloat16, device=DEV)
    kc2 = mxa.quantize(k2, "hd")
    with pytest.raises(mxa.MxattnError, match="partial slots"):
        mxa.decode(_query(q), kc2, kc2, ctx, split_len=split)


def test_decode_32k_batch32_full_size():
    """Batch 32, 32/8 heads, D=128, ctx 32768, split 2048: cache codes of the
    sampled KV heads bit-exact, 12 sampled (b, hq) outputs vs the oracle."""
    d = synth.long_decode(device=DEV)
    print("decode 32K batch 32 full size", flush=True)
    kc, vc = _cache(d["k"], d["v"])
    qh = _query(d["q"])
    out, lse = mxa.decode(qh, kc, vc, d["ctx_len"], split_len=2048, return_lse=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    pairs = [(int(rng.integers(32)), int(rng.integers(32))) for _ in range(12)]
    for (b, h) in pairs[:3]:
        kv = h // 4
        oc = oracle_quantize(host_f64(d["k"][b:b + 1, kv:kv + 1]), "hd")
        sub = mxa.MX(kc.codes[b:b + 1, kv:kv + 1], kc.scales[b:b + 1, kv:kv + 1], (1, 1, 32768, 128), "hd")
        assert_codes_equal(sub, *oc, f"cache b{b} kv{kv}")
    ref = _oracle_pair(d["q"], d["k"], d["v"], d["ctx_len"].cpu().numpy(), pairs)
    _compare(out, lse, ref, "decode 32K batch 32")
    # The same cache as a shuffled pool of 64-token pages, split 4096.
    del d["k"], d["v"]
    ref4 = mxa.decode(qh, kc, vc, d["ctx_len"], split_len=4096)
    kp, table = _page_pool(kc, 64, d["ctx_len"], seed=11, spare=0)
    del kc
    vp, _ = _page_pool(vc, 64, d["ctx_len"], seed=11, spare=0)
    del vc
    print("decode 32K batch 32, paged (64-token pages)", flush=True)
    paged = mxa.decode_paged(qh, kp, vp, table, d["ctx_len"], split_len=4096)
    torch.cuda.synchronize()
    assert torch.equal(ref4, paged)


def test_hybrid_decode_32k_batch8_full_size():
    """Batch 8, 32/8 heads, ctx 32768, heavy-tailed column bias, window 128,
    1632 selected tokens per KV head (seeded), rest MXFP4."""
    d = synth.hybrid_decode(device=DEV)
    print("hybrid decode 32K batch 8 full size", flush=True)
    kc, vc = _cache(d["k"], d["v"])
    qh = _query(d["q"])
    hy, sets = _hybrid_inputs(d["q"], d["k"], d["v"], d["ctx_len"].cpu().numpy(), 128, 1632, 1632, 9)
    out, lse = mxa.decode(qh, kc, vc, d["ctx_len"], split_len=2048, hybrid=hy, q_bf16=d["q"].contiguous(),
                          return_lse=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(4)
    pairs = [(int(rng.integers(8)), int(rng.integers(32))) for _ in range(8)]
    ref = _oracle_pair(d["q"], d["k"], d["v"], d["ctx_len"].cpu().numpy(), pairs, hybrid_sets=sets, q_bf=d["q"])
    _compare(out, lse, ref, "hybrid 32K batch 8")


# ------------------------------------------------------------------ selection
@pytest.mark.parametrize("tcap", [5000, 40000])
def test_topk_exact_on_given_masses(tcap):
    """R = 0: only the top-k runs, on integer-valued masses with many ties;
    the indices must equal the oracle's exactly.  Contexts above 32K take the
    second register layout of the selection."""
    rng = np.random.default_rng(41)
    b, hkv = 3, 2
    cm = rng.integers(0, 50, size=(b, hkv, tcap)).astype(np.float32)
    ctx = np.array([tcap, (3 * tcap) // 5 + 1, 129], dtype=np.int32)
    kc = mxa.empty_mx((b, hkv, tcap, 128), "hd", DEV)
    col = torch.from_numpy(cm).to(DEV)
    idx, n = mxa.select_vertical(None, kc, torch.from_numpy(ctx).to(DEV), col, window=128,
                                 rho_num=5, rho_den=100)
    torch.cuda.synchronize()
    for bb in range(b):
        for h in range(hkv):
            want = select.topk_vertical(cm[bb, h], int(ctx[bb]), 128, 5, 100)
            got = idx[bb, h, : int(n[bb, h])].cpu().numpy()
            np.testing.assert_array_equal(got, want)
            assert (idx[bb, h, int(n[bb, h]):].cpu().numpy() == -1).all()


@pytest.mark.parametrize("kind", ["equal", "near_equal", "uniform", "zeros", "rho0"])
def test_topk_exact_on_edge_masses(kind):
    """R = 0, top-k only, indices equal to the oracle's: every mass equal (all
    ties), masses that differ only in their lowest mantissa bits (the
    threshold is decided by the last byte), uniform floats, all zeros, and
    rho = 0 (nothing selected)."""
    rng = np.random.default_rng(43)
    b, hkv, tcap = 2, 2, 9000
    if kind == "equal":
        cm = np.full((b, hkv, tcap), 0.375, dtype=np.float32)
    elif kind == "near_equal":
        base = np.float32(1.0).view(np.uint32)
        cm = (base + rng.integers(0, 700, size=(b, hkv, tcap)).astype(np.uint32)).view(np.float32)
    elif kind == "uniform":
        cm = rng.uniform(0, 3, size=(b, hkv, tcap)).astype(np.float32)
    else:
        cm = np.zeros((b, hkv, tcap), dtype=np.float32)
    num = 0 if kind == "rho0" else 7
    ctx = np.array([tcap, 4000], dtype=np.int32)
    kc = mxa.empty_mx((b, hkv, tcap, 128), "hd", DEV)
    col = torch.from_numpy(cm).to(DEV)
    idx, n = mxa.select_vertical(None, kc, torch.from_numpy(ctx).to(DEV), col, window=64,
                                 rho_num=num, rho_den=100)
    torch.cuda.synchronize()
    for bb in range(b):
        for h in range(hkv):
            want = select.topk_vertical(cm[bb, h], int(ctx[bb]), 64, num, 100)
            got = idx[bb, h, : int(n[bb, h])].cpu().numpy()
            np.testing.assert_array_equal(got, want, err_msg=f"{kind} b{bb} h{h}")
            assert (idx[bb, h, int(n[bb, h]):].cpu().numpy() == -1).all()


@pytest.mark.parametrize("kind", ["uniform", "ties"])
def test_topk_exact_large_k_and_unaligned_rows(kind):
    """R = 0, top-k only, indices equal to the oracle's: a 64K context with
    rho = 60% selects more than 32768 keys, past what the kernel stages in
    LDS, so the indices are written straight to the output; the mass rows
    are 16-byte misaligned (Tcap odd), which takes the word-wise loads."""
    rng = np.random.default_rng(47)
    b, hkv, tcap = 2, 2, 65533
    if kind == "uniform":
        cm = rng.uniform(0, 3, size=(b, hkv, tcap)).astype(np.float32)
    else:
        cm = rng.integers(0, 6, size=(b, hkv, tcap)).astype(np.float32)
    ctx = np.array([tcap, 40001], dtype=np.int32)
    kc = mxa.empty_mx((b, hkv, tcap, 64), "hd", DEV)
    col = torch.from_numpy(cm).to(DEV)
    print(f"top-k large k {kind}", flush=True)
    idx, n = mxa.select_vertical(None, kc, torch.from_numpy(ctx).to(DEV), col, window=100,
                                 rho_num=60, rho_den=100)
    torch.cuda.synchronize()
    assert int(n[0, 0]) > 32768
    for bb in range(b):
        for h in range(hkv):
            want = select.topk_vertical(cm[bb, h], int(ctx[bb]), 100, 60, 100)
            got = idx[bb, h, : int(n[bb, h])].cpu().numpy()
            np.testing.assert_array_equal(got, want, err_msg=f"{kind} b{bb} h{h}")
            assert (idx[bb, h, int(n[bb, h]):].cpu().numpy() == -1).all()


@pytest.mark.parametrize("b,hq,hkv,r,d,tcap,ctxs", [
    (2, 8, 1, 40, 64, 3000, (3000, 1777)),   # 320 queries: 16-group state, operands read from LDS
    (1, 4, 2, 17, 128, 9000, (8999,)),       # 34 queries: partial groups, operands in registers
    (3, 4, 1, 64, 128, 1100, (1100, 129, 700)),
])
def test_select_column_mass_short_contexts(b, hq, hkv, r, d, tcap, ctxs):
    """Column mass and top 5% against the oracle where the stats chunks and
    column-mass blocks shrink for short contexts (256-512-key chunks,
    128-key blocks), on ragged contexts, with 16 query groups, partial
    groups and D = 64."""
    g = torch.Generator(device=DEV).manual_seed(1000 + tcap)
    k = torch.randn((b, hkv, tcap, d), generator=g, device=DEV).to(torch.bfloat16)
    q = torch.randn((b, hq, r, d), generator=g, device=DEV).to(torch.bfloat16)
    kc, qr = mxa.quantize(k, "hd"), mxa.quantize(q, "hd")
    ctx = torch.tensor(ctxs, dtype=torch.int32, device=DEV)
    col = torch.zeros((b, hkv, tcap), dtype=torch.float32, device=DEV)
    print(f"select short contexts b={b} hq={hq} hkv={hkv} r={r} d={d} tcap={tcap}", flush=True)
    idx, n = mxa.select_vertical(qr, kc, ctx, col, window=32)
    torch.cuda.synchronize()
    kd = oracle_dequant(*oracle_quantize(host_f64(k), "hd"), "hd")
    qd = oracle_dequant(*oracle_quantize(host_f64(q), "hd"), "hd")
    grp = hq // hkv
    for bb in range(b):
        c = int(ctxs[bb])
        for h in range(hkv):
            ocm = select.colmass_update(np.zeros(tcap), qd[bb, grp * h:grp * (h + 1)].reshape(-1, d), kd[bb, h], c)
            np.testing.assert_allclose(col[bb, h].cpu().numpy(), ocm, rtol=2e-4, atol=1e-7,
                                       err_msg=f"column mass b{bb} h{h}")
            check_selection(idx[bb, h, : int(n[bb, h])].cpu().numpy(), int(n[bb, h]), ocm, c, 32, 5, 100,
                            f"select b{bb} h{h}")


def test_select_vertical_32k_batch8():
    """col_mass from 64 recent queries x 4 heads per KV head over ctx 32768,
    then the top 5% of the non-window prefix; two calls accumulate."""
    d = synth.hybrid_decode(device=DEV)
    print("select 32K batch 8 full size", flush=True)
    kc = mxa.quantize(d["k"], "hd")
    qr = mxa.quantize(d["q_recent"], "hd")
    col = torch.zeros((8, 8, 32768), dtype=torch.float32, device=DEV)
    idx, n = mxa.select_vertical(qr, kc, d["ctx_len"], col, window=128)
    torch.cuda.synchronize()
    col1 = col.clone()
    idx2, n2 = mxa.select_vertical(qr, kc, d["ctx_len"], col, window=128)
    torch.cuda.synchronize()
    for (b, h) in [(0, 0), (3, 5), (7, 7)]:
        kk = host_f64(d["k"][b:b + 1, h:h + 1])
        kd = oracle_dequant(*oracle_quantize(kk, "hd"), "hd")[0, 0]
        qq = host_f64(d["q_recent"][b:b + 1, 4 * h:4 * h + 4])
        qd = oracle_dequant(*oracle_quantize(qq, "hd"), "hd")[0].reshape(-1, 128)
        ocm = select.colmass_update(np.zeros(32768), qd, kd, 32768)
        np.testing.assert_allclose(col1[b, h].cpu().numpy(), ocm, rtol=2e-4, atol=1e-7)
        np.testing.assert_allclose(col[b, h].cpu().numpy(), 2 * ocm, rtol=2e-4, atol=2e-7)
        check_selection(idx[b, h, : int(n[b, h])].cpu().numpy(), int(n[b, h]), ocm, 32768, 128, 5, 100,
                         f"select b{b} h{h}")
        # The mass actually concentrates on few keys (vertical lines).
        top = np.sort(ocm[:32640])[::-1]
        frac = top[:1632].sum() / top.sum()
        print(f"  b{b} h{h}: top-5% non-window mass fraction {frac:.3f}", flush=True)


def test_decode_degenerate_zero_query_gives_mean():
    """q = 0: all logits 0, so the output is the mean of the first ctx
    dequantised V rows (closed form) and lse = ln(ctx)."""
    g = torch.Generator(device=DEV).manual_seed(83)
    b, hq, hkv, tcap, d = 2, 4, 2, 1000, 128
    q = torch.zeros((b, hq, d), device=DEV, dtype=torch.bfloat16)
    k = torch.randn((b, hkv, tcap, d), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((b, hkv, tcap, d), generator=g, device=DEV).to(torch.bfloat16)
    ctx = torch.tensor([1000, 77], dtype=torch.int32, device=DEV)
    kc, vc = _cache(k, v)
    out, lse = mxa.decode(_query(q), kc, vc, ctx, split_len=256, return_lse=True)
    torch.cuda.synchronize()
    vd = oracle_dequant(*oracle_quantize(host_f64(v), "hd"), "hd")
    for bb in range(b):
        c = int(ctx[bb])
        for h in range(hq):
            np.testing.assert_allclose(out[bb, h].cpu().numpy(), vd[bb, h // 2, :c].mean(axis=0), atol=1e-5, rtol=0)
            assert abs(float(lse[bb, h]) - np.log(c)) < 1e-5


@pytest.mark.parametrize("d", [128, 64])
def test_gather_rows_matches_host_indexing(d):
    """mxattn_gather_rows against numpy fancy indexing on host copies, bit for
    bit: strided K (a view of a wider cache), ragged n_sel, indices outside
    [0, T) (zero rows), rows past n_sel left as they were."""
    g = torch.Generator(device=DEV).manual_seed(95)
    b, h, t, m = 2, 3, 1000, 40
    kbig = torch.randn((b, h, t + 24, d), generator=g, device=DEV).to(torch.bfloat16)
    k = kbig[:, :, 10:10 + t]                      # token-strided view
    v = torch.randn((b, h, t, d), generator=g, device=DEV).to(torch.bfloat16)
    rng = np.random.default_rng(96)
    idx = rng.integers(0, t, size=(b, h, m)).astype(np.int32)
    idx[0, 1, 3] = -1
    idx[1, 2, 5] = t + 7
    nsel = np.array([[m, 17, 0], [1, m, 33]], dtype=np.int32)
    ko = torch.full((b, h, m, d), 7.0, dtype=torch.bfloat16, device=DEV)
    vo = torch.full_like(ko, -3.0)
    print(f"gather rows d={d}", flush=True)
    mxa.gather_rows(k, v, torch.from_numpy(idx).to(DEV), torch.from_numpy(nsel).to(DEV), ko, vo)
    torch.cuda.synchronize()
    kh = k.cpu().view(torch.int16).numpy()
    vh = v.cpu().view(torch.int16).numpy()
    gk, gv = ko.cpu().view(torch.int16).numpy(), vo.cpu().view(torch.int16).numpy()
    seven = torch.tensor(7.0, dtype=torch.bfloat16).view(torch.int16).item()
    mthree = torch.tensor(-3.0, dtype=torch.bfloat16).view(torch.int16).item()
    for bb in range(b):
        for hh in range(h):
            n = int(nsel[bb, hh])
            for i in range(m):
                tt = int(idx[bb, hh, i])
                if i >= n:
                    assert (gk[bb, hh, i] == seven).all() and (gv[bb, hh, i] == mthree).all()
                elif 0 <= tt < t:
                    np.testing.assert_array_equal(gk[bb, hh, i], kh[bb, hh, tt])
                    np.testing.assert_array_equal(gv[bb, hh, i], vh[bb, hh, tt])
                else:
                    assert (gk[bb, hh, i] == 0).all() and (gv[bb, hh, i] == 0).all()
