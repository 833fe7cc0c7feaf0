"""GPU parity of the MXFP4 prefill against the float64 oracle on the same
quantised operands: max |gpu - oracle| <= 2e-3 per row, plus the oracle's
per-row float32 rounding envelope (rows whose P elements sit within float32
reach of an E2M1 midpoint or scale boundary, where both codes are correct)."""

import numpy as np
import pytest
import torch

import bit_microscaled_flashattention_amd as mxa
import synth
from oracle import attention, mx, rotate, smooth
from tests.helpers import (assert_codes_equal, check_prefill, head_slice, host_f64, oracle_dequant,
                           oracle_quantize)

pytestmark = pytest.mark.gpu
DEV = "cuda"
ATOL = 2e-3


def _run_case(q, k, v, *, causal, kv_tile=128, p_rule="ocp", qkv_rule="ocp", l_from_quantized=True,
              rows=None, q_scale=None, k_scale=None, out_dtype=torch.float32, heads=None, what="",
              hadamard=False, hybrid=None):
    """Quantise on the GPU, run prefill on every head, then check codes and
    outputs against the oracle on ``heads`` (query heads, default all) and
    ``rows`` (dict hq -> row indices, default all rows)."""
    print(f"prefill case {what}: q{tuple(q.shape)} k{tuple(k.shape)} causal={causal} "
          f"tile={kv_tile} p={p_rule}", flush=True)
    qh = mxa.quantize(q, "hd", chan_scale=q_scale, rule=qkv_rule, hadamard=hadamard)
    kh = mxa.quantize(k, "hd", chan_scale=k_scale, rule=qkv_rule, hadamard=hadamard)
    vh = mxa.quantize(v, "key", rule=qkv_rule)
    if hybrid is None:
        out, lse = mxa.prefill(qh, kh, vh, causal=causal, kv_tile=kv_tile, p_rule=p_rule,
                               l_from_quantized=l_from_quantized, out_dtype=out_dtype, return_lse=True)
    else:
        assert causal
        out, lse = mxa.prefill_hybrid(qh, kh, vh, q, k, v, hybrid["window"], hybrid.get("idx"),
                                      hybrid.get("n_sel"), kv_tile=kv_tile, p_rule=p_rule,
                                      l_from_quantized=l_from_quantized, out_dtype=out_dtype, return_lse=True)
    torch.cuda.synchronize()
    return check_prefill(q, k, v, qh, kh, vh, out, lse, causal=causal, kv_tile=kv_tile, p_rule=p_rule,
                         qkv_rule=qkv_rule, l_from_quantized=l_from_quantized, rows=rows, q_scale=q_scale,
                         k_scale=k_scale, heads=heads, what=what, hadamard=hadamard, hybrid=hybrid)


def test_tiny_noncausal_128x64():
    """Batch 1, 1 head, S=128, D=64, fp16, non-causal, single key tile."""
    d = synth.tiny(device=DEV)
    _run_case(d["q"], d["k"], d["v"], causal=False, what="tiny 128x64")


@pytest.mark.parametrize("kv_tile", [64, 128, 256])
@pytest.mark.parametrize("causal", [True, False])
def test_gqa_ragged_tiles(kv_tile, causal):
    g = torch.Generator(device=DEV).manual_seed(21)
    s = 333
    q = torch.randn((1, 4, s, 128), generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn((1, 2, s, 128), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((1, 2, s, 128), generator=g, device=DEV).to(torch.bfloat16)
    _run_case(q, k, v, causal=causal, kv_tile=kv_tile, what=f"gqa ragged tile={kv_tile}")


def test_non_causal_gqa_whole_pairs_per_xcd_ragged():
    """Non-causal launch whose (batch, KV head) pairs split evenly over the 8
    XCDs, so each XCD runs one pair's query blocks after another: GQA group
    of 4, a ragged query length (3 blocks, the last one partial) and a longer
    key length, every row against the oracle."""
    g = torch.Generator(device=DEV).manual_seed(23)
    q = torch.randn((2, 16, 300, 128), generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn((2, 4, 520, 128), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((2, 4, 520, 128), generator=g, device=DEV).to(torch.bfloat16)
    _run_case(q, k, v, causal=False, what="non-causal 8 pairs ragged")


def test_rectangular_non_causal_d64_batch2():
    g = torch.Generator(device=DEV).manual_seed(22)
    q = torch.randn((2, 2, 200, 64), generator=g, device=DEV).to(torch.float16)
    k = torch.randn((2, 1, 417, 64), generator=g, device=DEV).to(torch.float16)
    v = torch.randn((2, 1, 417, 64), generator=g, device=DEV).to(torch.float16)
    _run_case(q, k, v, causal=False, what="rect d64")


@pytest.mark.parametrize("rule", ["uos", "ocp"])
def test_uos_everywhere_and_baseline_normaliser(rule):
    g = torch.Generator(device=DEV).manual_seed(23)
    q = (torch.randn((1, 2, 260, 128), generator=g, device=DEV) * 2).to(torch.bfloat16)
    k = torch.randn((1, 2, 260, 128), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((1, 2, 260, 128), generator=g, device=DEV).to(torch.bfloat16)
    _run_case(q, k, v, causal=True, p_rule=rule, qkv_rule=rule, what=f"{rule} all")
    _run_case(q, k, v, causal=True, p_rule=rule, l_from_quantized=False, what=f"{rule} baseline-l")


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float16])
def test_low_precision_output(out_dtype):
    g = torch.Generator(device=DEV).manual_seed(24)
    q = torch.randn((1, 2, 130, 128), generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn((1, 2, 130, 128), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((1, 2, 130, 128), generator=g, device=DEV).to(torch.bfloat16)
    _run_case(q, k, v, causal=True, out_dtype=out_dtype, what=f"out {out_dtype}")


def test_single_token_and_short():
    g = torch.Generator(device=DEV).manual_seed(25)
    for s in (1, 31, 33):
        q = torch.randn((1, 1, s, 128), generator=g, device=DEV).to(torch.bfloat16)
        k = torch.randn((1, 1, s, 128), generator=g, device=DEV).to(torch.bfloat16)
        v = torch.randn((1, 1, s, 128), generator=g, device=DEV).to(torch.bfloat16)
        _run_case(q, k, v, causal=True, what=f"s={s}")


def _sample_rows(seq, n, seed, heads):
    """Rows 0, 1, 2, seq-1 and n distinct others, per head."""
    rng = np.random.default_rng(seed)
    return {h: np.sort(np.concatenate([[0, 1, 2, seq - 1], rng.choice(np.arange(3, seq - 1), size=n,
                                                                       replace=False)]))
            for h in heads}


def test_gqa_prefill_4k_causal_sampled_rows():
    """Causal GQA 32/8 heads, S=4096, D=128, outlier K channels, static
    Smooth-QK from the calibration slice; all codes compared, 24 sampled rows
    per head compared with the oracle."""
    d = synth.gqa_prefill(device=DEV)
    qs, ks = mxa.smooth_calibrate(d["q_cal"], d["k_cal"])
    rows = _sample_rows(4096, 20, 5, range(32))
    _run_case(d["q"], d["k"], d["v"], causal=True, rows=rows, q_scale=qs, k_scale=ks,
              what="4K causal GQA full size")


def test_diffusion_prefill_sampled_rows():
    """Non-causal, 24 heads, S=32768, UOS on Q, K, V and P: all heads run,
    three heads and ten rows each are compared with the oracle."""
    d = synth.diffusion(device=DEV)
    heads = [0, 7, 23]
    rows = _sample_rows(32768, 6, 6, heads)
    _run_case(d["q"], d["k"], d["v"], causal=False, p_rule="uos", qkv_rule="uos", rows=rows,
              heads=heads, what="video diffusion full size")


@pytest.mark.parametrize("shape", [(1, 32, 8, 4096), (2, 16, 8, 4096), (1, 64, 8, 2048)])
def test_causal_schedule_matches_per_head_launches(shape):
    """Causal launches whose query blocks fill every CU exactly twice over run
    two blocks per workgroup (heavier pairs first).  Rows are independent, so
    output and lse equal, bit for bit, separate launches over each KV head's
    group (which are too small to be paired)."""
    b, hq, hkv, s = shape
    g = torch.Generator(device=DEV).manual_seed(27)
    print(f"paired schedule {shape}", flush=True)
    q = torch.randn((b, hq, s, 128), generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn((b, hkv, s, 128), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((b, hkv, s, 128), generator=g, device=DEV).to(torch.bfloat16)
    qh, kh, vh = mxa.quantize(q, "hd"), mxa.quantize(k, "hd"), mxa.quantize(v, "key")
    out, lse = mxa.prefill(qh, kh, vh, causal=True, return_lse=True)
    grp = hq // hkv
    for bi in range(b):
        for h in range(hkv):
            qs = mxa.quantize(q[bi:bi + 1, h * grp:(h + 1) * grp].contiguous(), "hd")
            ks = mxa.quantize(k[bi:bi + 1, h:h + 1].contiguous(), "hd")
            vs = mxa.quantize(v[bi:bi + 1, h:h + 1].contiguous(), "key")
            o1, l1 = mxa.prefill(qs, ks, vs, causal=True, return_lse=True)
            assert torch.equal(o1[0], out[bi, h * grp:(h + 1) * grp]), (bi, h)
            assert torch.equal(l1[0], lse[bi, h * grp:(h + 1) * grp]), (bi, h)


def test_hybrid_causal_schedule_matches_per_head_launches():
    """The hybrid prefill on the paired schedule (4K, 32/8 heads: one round
    of two workgroups per CU) equals, bit for bit, separate hybrid launches
    over each KV head's group."""
    b, hq, hkv, s, w, n_sel = 1, 32, 8, 4096, 128, 150
    g = torch.Generator(device=DEV).manual_seed(31)
    print("paired schedule, hybrid prefill 4K", flush=True)
    q = torch.randn((b, hq, s, 128), generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn((b, hkv, s, 128), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((b, hkv, s, 128), generator=g, device=DEV).to(torch.bfloat16)
    rng = np.random.default_rng(31)
    idx = torch.from_numpy(np.stack([np.sort(rng.choice(s - w, size=n_sel, replace=False))
                                     for _ in range(hkv)]).astype(np.int32)[None]).to(DEV)
    nsel = torch.full((b, hkv), n_sel, dtype=torch.int32, device=DEV)
    qh, kh, vh = mxa.quantize(q, "hd"), mxa.quantize(k, "hd"), mxa.quantize(v, "key")
    out, lse = mxa.prefill_hybrid(qh, kh, vh, q, k, v, w, idx, nsel, return_lse=True)
    grp = hq // hkv
    for h in range(hkv):
        qs_ = q[:, h * grp:(h + 1) * grp].contiguous()
        ks_, vs_ = k[:, h:h + 1].contiguous(), v[:, h:h + 1].contiguous()
        o1, l1 = mxa.prefill_hybrid(mxa.quantize(qs_, "hd"), mxa.quantize(ks_, "hd"), mxa.quantize(vs_, "key"),
                                    qs_, ks_, vs_, w, idx[:, h:h + 1].contiguous(), nsel[:, h:h + 1].contiguous(),
                                    return_lse=True)
        assert torch.equal(o1[0], out[0, h * grp:(h + 1) * grp]), h
        assert torch.equal(l1[0], lse[0, h * grp:(h + 1) * grp]), h


def test_deterministic_and_launch_order_independent():
    g = torch.Generator(device=DEV).manual_seed(26)
    q = torch.randn((1, 8, 512, 128), generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn((1, 2, 512, 128), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((1, 2, 512, 128), generator=g, device=DEV).to(torch.bfloat16)
    qh, kh, vh = mxa.quantize(q), mxa.quantize(k), mxa.quantize(v, "key")
    a = mxa.prefill(qh, kh, vh, causal=True)
    b = mxa.prefill(qh, kh, vh, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("d", [128, 64])
def test_prefill_hadamard_rotated_qk(d):
    """Q and K rotated by the Walsh-Hadamard transform before MXFP4 (codes
    bit-exact with the oracle's float32 transform), with Smooth-QK first."""
    g = torch.Generator(device=DEV).manual_seed(51)
    q = torch.randn((1, 4, 300, d), generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn((1, 2, 300, d), generator=g, device=DEV).to(torch.bfloat16)
    k[:, :, :, 5] *= 12
    v = torch.randn((1, 2, 300, d), generator=g, device=DEV).to(torch.bfloat16)
    qs = torch.exp(0.3 * torch.randn((4, d), generator=g, device=DEV)).float()
    ks = torch.exp(0.3 * torch.randn((2, d), generator=g, device=DEV)).float()
    _run_case(q, k, v, causal=True, q_scale=qs, k_scale=ks, hadamard=True, what=f"hadamard d={d}")


def test_hadamard_rotation_cuts_error_on_key_outliers():
    """On the outlier workload (4 K channels x12 per KV head) the rotation
    brings the MXFP4 prefill closer to float64 attention on the unquantised
    inputs (measured on 4 query heads, 512 rows)."""
    d = synth.gqa_prefill(device=DEV, seq=512)
    outs = {}
    for rot in (False, True):
        qh = mxa.quantize(d["q"], "hd", hadamard=rot)
        kh = mxa.quantize(d["k"], "hd", hadamard=rot)
        vh = mxa.quantize(d["v"], "key")
        outs[rot] = mxa.prefill(qh, kh, vh, causal=True).cpu().numpy()
    torch.cuda.synchronize()
    err = {False: [], True: []}
    for h in (0, 9, 18, 27):
        kv = h // 4
        ref = attention.prefill_head(host_f64(d["q"][0, h]), host_f64(d["k"][0, kv]), host_f64(d["v"][0, kv]),
                                     causal=True, quantize_p=False)["out"]
        for rot in (False, True):
            err[rot].append(np.abs(outs[rot][0, h] - ref).mean())
    e0, e1 = float(np.mean(err[False])), float(np.mean(err[True]))
    print(f"  mean |out - exact|: plain {e0:.3e}, rotated {e1:.3e}", flush=True)
    assert e1 < e0


def _sel_sets(b, hkv, s, n, max_sel, seed, lo=0):
    """Seeded ascending selected sets per (batch, KV head), -1 padded."""
    rng = np.random.default_rng(seed)
    idx = np.full((b, hkv, max_sel), -1, dtype=np.int32)
    nsel = np.zeros((b, hkv), dtype=np.int32)
    for bi in range(b):
        for h in range(hkv):
            k = min(n, s - lo) if h % 2 == 0 else min(n // 2, s - lo)
            pick = np.sort(rng.choice(np.arange(lo, s), size=k, replace=False))
            idx[bi, h, :k] = pick
            nsel[bi, h] = k
    return torch.from_numpy(idx).to(DEV), torch.from_numpy(nsel).to(DEV)


@pytest.mark.parametrize("d, kv_tile, window, n_sel", [
    (128, 128, 64, 40), (128, 64, 200, 17), (128, 256, 1, 90), (64, 128, 130, 33), (128, 128, 0, 60),
])
def test_hybrid_prefill_parity(d, kv_tile, window, n_sel):
    """bf16 window and selected keys after the 4-bit tiles, one softmax:
    every row of a ragged multi-block case against the oracle."""
    g = torch.Generator(device=DEV).manual_seed(70 + d + window)
    b, hq, hkv, s = 2, 4, 2, 700
    q = torch.randn((b, hq, s, d), generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn((b, hkv, s, d), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((b, hkv, s, d), generator=g, device=DEV).to(torch.bfloat16)
    idx, nsel = _sel_sets(b, hkv, s, n_sel, 96, seed=window + n_sel)
    _run_case(q, k, v, causal=True, kv_tile=kv_tile, hybrid={"window": window, "idx": idx, "n_sel": nsel},
              what=f"hybrid d={d} tile={kv_tile} W={window} n={n_sel}")


@pytest.mark.parametrize("p_rule, lq", [("uos", True), ("ocp", False)])
def test_hybrid_prefill_rules_and_baseline_normaliser(p_rule, lq):
    g = torch.Generator(device=DEV).manual_seed(77)
    q = (torch.randn((1, 2, 333, 128), generator=g, device=DEV) * 1.5).to(torch.bfloat16)
    k = torch.randn((1, 1, 333, 128), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((1, 1, 333, 128), generator=g, device=DEV).to(torch.bfloat16)
    idx, nsel = _sel_sets(1, 1, 333, 25, 32, seed=3)
    _run_case(q, k, v, causal=True, p_rule=p_rule, l_from_quantized=lq,
              hybrid={"window": 48, "idx": idx, "n_sel": nsel}, what=f"hybrid p={p_rule} lq={lq}")


def test_hybrid_prefill_limits():
    """Window 0 and no selected keys: the plain kernel's output bit for bit.
    Window >= S: attention on the bf16 rows alone (oracle, no 4-bit key)."""
    g = torch.Generator(device=DEV).manual_seed(78)
    q = torch.randn((1, 4, 300, 128), generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn((1, 2, 300, 128), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((1, 2, 300, 128), generator=g, device=DEV).to(torch.bfloat16)
    qh, kh, vh = mxa.quantize(q), mxa.quantize(k), mxa.quantize(v, "key")
    plain, lp = mxa.prefill(qh, kh, vh, causal=True, return_lse=True)
    empty = torch.zeros((1, 2, 4), dtype=torch.int32, device=DEV)
    hy0, l0 = mxa.prefill_hybrid(qh, kh, vh, q, k, v, 0, empty, torch.zeros((1, 2), dtype=torch.int32, device=DEV),
                                 return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(plain, hy0) and torch.equal(lp, l0)
    _run_case(q, k, v, causal=True, hybrid={"window": 300}, what="hybrid all-bf16 window")


def test_hybrid_prefill_cuts_error_on_heavy_columns():
    """Keys that every query attends strongly (vertical lines) held in bf16:
    the output moves towards float64 attention on the bf16 inputs."""
    g = torch.Generator(device=DEV).manual_seed(79)
    b, hq, hkv, s, dd = 1, 4, 2, 1024, 128
    q = torch.randn((b, hq, s, dd), generator=g, device=DEV)
    k = torch.randn((b, hkv, s, dd), generator=g, device=DEV)
    heavy = torch.tensor([3, 100, 257, 600], device=DEV)
    dirn = q.mean(dim=(1, 2))[:, None, :]            # a shared query direction
    k[:, :, heavy] += 24.0 * dirn[:, :, None, :] / dirn.norm()
    q = q + 2.0 * dirn[:, :, None, :] / dirn.norm()
    q, k = q.to(torch.bfloat16), k.to(torch.bfloat16)
    v = torch.randn((b, hkv, s, dd), generator=g, device=DEV).to(torch.bfloat16)
    qh, kh, vh = mxa.quantize(q), mxa.quantize(k), mxa.quantize(v, "key")
    idx = heavy.to(torch.int32).repeat(b, hkv, 1).contiguous()
    nsel = torch.full((b, hkv), 4, dtype=torch.int32, device=DEV)
    plain = mxa.prefill(qh, kh, vh, causal=True).cpu().numpy()
    hyb = mxa.prefill_hybrid(qh, kh, vh, q, k, v, 64, idx, nsel).cpu().numpy()
    torch.cuda.synchronize()
    e_p, e_h = [], []
    for h in range(hq):
        ref = attention.prefill_head(host_f64(q[0, h]), host_f64(k[0, h // 2]), host_f64(v[0, h // 2]),
                                     causal=True, quantize_p=False)["out"]
        e_p.append(np.abs(plain[0, h] - ref).mean())
        e_h.append(np.abs(hyb[0, h] - ref).mean())
    print(f"  mean |out - exact|: 4-bit {np.mean(e_p):.3e}, hybrid {np.mean(e_h):.3e}", flush=True)
    assert np.mean(e_h) < 0.8 * np.mean(e_p)


def test_degenerate_zero_query_gives_running_mean():
    """All logits 0: every P~ is 1, so P_hat = 1 exactly and the causal output
    of row i is the mean of the dequantised V rows 0..i (closed form, no
    attention code involved); lse = ln(i + 1)."""
    g = torch.Generator(device=DEV).manual_seed(81)
    s, d = 300, 128
    q = torch.zeros((1, 2, s, d), device=DEV, dtype=torch.bfloat16)
    k = torch.randn((1, 1, s, d), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((1, 1, s, d), generator=g, device=DEV).to(torch.bfloat16)
    qh, kh, vh = mxa.quantize(q), mxa.quantize(k), mxa.quantize(v, "key")
    for tile in (64, 128, 256):
        out, lse = mxa.prefill(qh, kh, vh, causal=True, kv_tile=tile, return_lse=True)
        torch.cuda.synchronize()
        vd = oracle_dequant(*oracle_quantize(host_f64(v), "key"), "key", n=s)[0, 0]
        mean = np.cumsum(vd, axis=0) / np.arange(1, s + 1)[:, None]
        for h in range(2):
            np.testing.assert_allclose(out[0, h].cpu().numpy(), mean, atol=1e-5, rtol=0)
            np.testing.assert_allclose(lse[0, h].cpu().numpy(), np.log(np.arange(1, s + 1)), atol=1e-5, rtol=0)


def test_degenerate_one_dominant_key_gives_its_row():
    """One key whose logit beats every other by far more than the fp32
    exponent range: the softmax is one-hot, so each row from that key on
    outputs that key's dequantised V row exactly."""
    g = torch.Generator(device=DEV).manual_seed(82)
    s, d, hot = 256, 128, 37
    q = torch.randn((1, 1, s, d), generator=g, device=DEV).abs().to(torch.bfloat16)
    k = (torch.randn((1, 1, s, d), generator=g, device=DEV) * 0.01).to(torch.bfloat16)
    k[0, 0, hot] = 400.0
    v = torch.randn((1, 1, s, d), generator=g, device=DEV).to(torch.bfloat16)
    qh, kh, vh = mxa.quantize(q), mxa.quantize(k), mxa.quantize(v, "key")
    out = mxa.prefill(qh, kh, vh, causal=True)
    torch.cuda.synchronize()
    vd = oracle_dequant(*oracle_quantize(host_f64(v), "key"), "key", n=s)[0, 0]
    o = out[0, 0].cpu().numpy()
    np.testing.assert_array_equal(o[hot:], np.broadcast_to(vd[hot], (s - hot, d)).astype(np.float32))
    _run_case(q, k, v, causal=True, what="one dominant key")
