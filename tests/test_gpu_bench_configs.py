"""GPU parity at the launch configurations bench.py times, against the oracle.

Each test issues the same library calls as the benchmark leg it names (same
quantiser launch, split length, query encoding, tile width and selection
procedure) on the same seeded workload, then compares sampled outputs with
the float64 oracle: codes and scales bit for bit, outputs within 2e-3 (plus
the oracle's rounding envelope for prefill rows, plus the output rounding
for 16-bit outputs).  Selected token sets fed to an attention call come from
the oracle's own selection, so no oracle input is taken from the GPU; the
GPU's selection is checked against the oracle's column mass separately.
"""

import numpy as np
import pytest
import torch

import bench
import bit_microscaled_flashattention_amd as mxa
import synth
from oracle import attention, mx, select, smooth
from tests.helpers import (assert_codes_equal, check_prefill, check_selection, host_f64, oracle_dequant,
                           oracle_quantize)

pytestmark = pytest.mark.gpu
DEV = "cuda"
ATOL = 2e-3


def _rows(seq, n, seed, heads, edges):
    """Per head: the given edge rows plus n distinct seeded others."""
    rng = np.random.default_rng(seed)
    edges = np.asarray(sorted(set(edges)))
    pool = np.setdiff1d(np.arange(seq), edges)
    return {h: np.sort(np.concatenate([edges, rng.choice(pool, size=n, replace=False)])) for h in heads}


# ------------------------------------------------------------ 4K causal GQA prefill
def _gqa_step(d, qs, ks):
    """The benchmark's prefill step: one quantiser launch for Q, K (with
    their Smooth-QK factors) and V, then the causal attention kernel."""
    qh, kh, vh = mxa.quantize_batch([dict(x=d["q"], chan_scale=qs), dict(x=d["k"], chan_scale=ks),
                                     dict(x=d["v"], layout="key")])
    return qh, kh, vh


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_prefill_4k_gqa_bench_step(out_dtype):
    """Batch 1, 32/8 heads, S 4096, D 128, outlier K channels, Smooth-QK,
    kv_tile 128 on the paired causal schedule; all codes, and 20 seeded rows
    plus the query-block edges of every head, fp32 and bf16 outputs."""
    d = synth.gqa_prefill(device=DEV)
    qs, ks = mxa.smooth_calibrate(d["q_cal"], d["k_cal"])
    print(f"bench prefill step, out {out_dtype}", flush=True)
    qh, kh, vh = _gqa_step(d, qs, ks)
    out, lse = mxa.prefill(qh, kh, vh, causal=True, kv_tile=bench.KV_TILE, out_dtype=out_dtype, return_lse=True)
    torch.cuda.synchronize()
    rows = _rows(4096, 20, 51, range(32), [0, 1, 2, 127, 128, 255, 256, 2047, 2048, 3968, 4095])
    check_prefill(d["q"], d["k"], d["v"], qh, kh, vh, out, lse, causal=True, kv_tile=bench.KV_TILE, rows=rows,
                  q_scale=qs, k_scale=ks, what=f"4K GQA bench step {out_dtype}")


def _oracle_colmass_selection(q_recent32, k32, ctx, window, rule=mx.RULE_OCP):
    """Oracle column mass and top-5% selection of one (batch, KV head) from
    float32 recent queries [G, R, D] and keys [T, D] (already smoothed)."""
    qd = oracle_dequant(*oracle_quantize(q_recent32[None].astype(np.float64), "hd", rule), "hd")[0]
    kd = oracle_dequant(*oracle_quantize(k32[None, None].astype(np.float64), "hd", rule), "hd")[0, 0]
    cm = select.colmass_update(np.zeros(k32.shape[0]), qd.reshape(-1, qd.shape[-1]), kd, ctx)
    return cm, select.topk_vertical(cm, ctx, window, 5, 100)


def test_hybrid_prefill_4k_gqa_bench_step():
    """The benchmark's hybrid prefill: the Smooth-QK step's operands, a
    128-key window per row and the top 5% of the non-window prefix by column
    mass of the last 64 (smoothed) queries, in bf16.  The GPU selection is
    checked against the oracle's column mass; the attention call then runs on
    the oracle's selection, sampled rows of eight heads against the oracle."""
    d = synth.gqa_prefill(device=DEV)
    S, W, HKV = 4096, bench.HYBRID_WINDOW, 8
    qs, ks = mxa.smooth_calibrate(d["q_cal"], d["k_cal"])
    qh, kh, vh = _gqa_step(d, qs, ks)
    qr = mxa.quantize(d["q"][:, :, S - 64:], "hd", chan_scale=qs)
    ctx = torch.tensor([S], dtype=torch.int32, device=DEV)
    col = torch.zeros((1, HKV, S), dtype=torch.float32, device=DEV)
    idx_g, n_g = mxa.select_vertical(qr, kh, ctx, col, window=W)
    torch.cuda.synchronize()
    q32 = smooth.apply(host_f64(d["q"][:, :, S - 64:]).astype(np.float32), qs.cpu().numpy())
    k32 = smooth.apply(host_f64(d["k"]).astype(np.float32), ks.cpu().numpy())
    k_sel = -(-(S - W) * 5 // 100)
    idx = np.full((1, HKV, k_sel), -1, dtype=np.int32)
    n = np.zeros((1, HKV), dtype=np.int32)
    for h in range(HKV):
        cm, sel = _oracle_colmass_selection(q32[0, 4 * h:4 * h + 4], k32[0, h], S, W)
        check_selection(idx_g[0, h, :int(n_g[0, h])].cpu().numpy(), int(n_g[0, h]), cm, S, W, 5, 100,
                        f"4K selection kv{h}")
        idx[0, h, :sel.size] = sel
        n[0, h] = sel.size
    idx_t, n_t = torch.from_numpy(idx).to(DEV), torch.from_numpy(n).to(DEV)
    print(f"hybrid prefill bench step: {n.ravel().tolist()} selected per KV head", flush=True)
    out, lse = mxa.prefill_hybrid(qh, kh, vh, d["q"], d["k"], d["v"], W, idx_t, n_t, kv_tile=bench.KV_TILE,
                                  return_lse=True)
    torch.cuda.synchronize()
    heads = [0, 5, 10, 15, 16, 21, 26, 31]
    rows = _rows(4096, 16, 52, heads, [0, 1, 127, 128, 129, 255, 256, 2048, 4095])
    check_prefill(d["q"], d["k"], d["v"], qh, kh, vh, out, lse, causal=True, kv_tile=bench.KV_TILE, rows=rows,
                  q_scale=qs, k_scale=ks, heads=heads, hybrid={"window": W, "idx": idx_t, "n_sel": n_t},
                  what="hybrid 4K GQA bench step")


# ------------------------------------------------- 32K non-causal diffusion prefill
@pytest.mark.parametrize("group", range(4))
def test_diffusion_prefill_bench_step(group):
    """Batch 1, 24 heads, S 32768, D 128, UOS (Qmax 7.25) on Q, K, V and P,
    one quantiser launch + the non-causal kernel, as the benchmark runs it.
    Heads 6*group .. 6*group+5: all K/V codes, and 256 rows of each head
    (245 seeded plus the query-block and tile edges) against the oracle."""
    d = synth.diffusion(device=DEV)
    print(f"diffusion bench step, heads {6 * group}..{6 * group + 5}", flush=True)
    qh, kh, vh = mxa.quantize_batch([dict(x=d["q"], rule="uos"), dict(x=d["k"], rule="uos"),
                                     dict(x=d["v"], layout="key", rule="uos")])
    out, lse = mxa.prefill(qh, kh, vh, causal=False, kv_tile=bench.KV_TILE, p_rule="uos", return_lse=True)
    torch.cuda.synchronize()
    heads = list(range(6 * group, 6 * group + 6))
    rows = _rows(32768, 245, 60 + group, heads, [0, 1, 127, 128, 255, 256, 16383, 16384, 32639, 32640, 32767])
    check_prefill(d["q"], d["k"], d["v"], qh, kh, vh, out, lse, causal=False, kv_tile=bench.KV_TILE,
                  p_rule="uos", qkv_rule="uos", rows=rows, heads=heads, q_rows_only=True,
                  what=f"diffusion heads {heads[0]}-{heads[-1]}")


# ------------------------------------------------------------------ 32K decode
def _oracle_kv(k, v, b, kv):
    kd = oracle_dequant(*oracle_quantize(host_f64(k[b:b + 1, kv:kv + 1]), "hd"), "hd")
    vd = oracle_dequant(*oracle_quantize(host_f64(v[b:b + 1, kv:kv + 1]), "hd"), "hd")
    return kd, vd


def _compare_group(out, lse, ref, b, kv, g, what):
    worst = 0.0
    for (_, hh), (ro, rl) in ref.items():
        h = kv * g + hh
        err = float(np.abs(out[b, h].cpu().numpy() - ro).max())
        worst = max(worst, err)
        assert err <= ATOL, f"{what}: (b={b}, h={h}) err {err:.3e}"
        assert abs(float(lse[b, h]) - rl) <= 1e-3, f"{what}: lse (b={b}, h={h})"
    return worst


def test_decode_32k_batch32_bench_call():
    """Batch 32, 32/8 heads, ctx 32768, the benchmark's one call per token:
    the bf16 query encoded inside the scan, the benchmark's split, merge.  The four
    query heads of four seeded (sequence, KV head) pairs against the oracle
    (query encoded by the oracle from the same bf16 values)."""
    d = synth.long_decode(device=DEV)
    kc, vc = mxa.quantize(d["k"], "hd"), mxa.quantize(d["v"], "hd")
    qbf = d["q"].contiguous()
    print(f"decode 32K batch 32 bench call, split {bench.DECODE_SPLIT}", flush=True)
    out, lse = mxa.decode(qbf, kc, vc, d["ctx_len"], split_len=bench.DECODE_SPLIT, return_lse=True)
    torch.cuda.synchronize()
    qd = oracle_dequant(*oracle_quantize(host_f64(d["q"][:, :, None, :]), "hd"), "hd")[:, :, 0]
    rng = np.random.default_rng(71)
    worst = 0.0
    for b, kv in [(0, 0), (int(rng.integers(32)), 3), (int(rng.integers(32)), 5), (31, 7)]:
        kd, vd = _oracle_kv(d["k"], d["v"], b, kv)
        ref = attention.decode(qd[b:b + 1, 4 * kv:4 * kv + 4], kd, vd, [32768])
        worst = max(worst, _compare_group(out, lse, ref, b, kv, 4, "decode bench call"))
    print(f"  worst |err| {worst:.3e} over 16 pairs", flush=True)


def test_hybrid_decode_32k_batch8_bench_call():
    """Batch 8, 32/8 heads, ctx 32768, heavy-tailed column bias: the
    benchmark's selection (column mass of 64 recent queries, top 5% of the
    non-window prefix, window 128) and its one hybrid decode call (bf16 query
    encoded in the scan for the 4-bit tokens, split 2752).  On three sampled
    (sequence, KV head) pairs the GPU selection is checked against the
    oracle's column mass, the decode runs on the oracle's selection there,
    and all four query heads are compared with the oracle."""
    d = synth.hybrid_decode(device=DEV)
    B, HQ, HKV, T, D, W = 8, 32, 8, 32768, 128, bench.HYBRID_WINDOW
    kc, vc = mxa.quantize(d["k"], "hd"), mxa.quantize(d["v"], "hd")
    qr = mxa.quantize(d["q_recent"], "hd")
    col = torch.zeros((B, HKV, T), dtype=torch.float32, device=DEV)
    idx, n = mxa.select_vertical(qr, kc, d["ctx_len"], col, window=W)
    torch.cuda.synchronize()
    picks = [(0, 0), (3, 5), (7, 2)]
    qrh = host_f64(d["q_recent"]).astype(np.float32)
    oracle_sets = {}
    for b, kv in picks:
        cm, sel = _oracle_colmass_selection(qrh[b, 4 * kv:4 * kv + 4], host_f64(d["k"][b, kv]).astype(np.float32),
                                            T, W)
        check_selection(idx[b, kv, :int(n[b, kv])].cpu().numpy(), int(n[b, kv]), cm, T, W, 5, 100,
                        f"32K selection b{b} kv{kv}")
        assert sel.size == idx.shape[-1]
        idx[b, kv] = torch.from_numpy(sel.astype(np.int32)).to(DEV)
        oracle_sets[(b, kv)] = sel
    # Gather the bf16 rows of the selected tokens and the window, as the benchmark does.
    k_sel, v_sel = mxa.gather_rows(d["k"], d["v"], idx, n)
    hy = {"idx": idx, "n_sel": n, "window": W, "k_sel": k_sel, "v_sel": v_sel,
          "k_win": d["k"][:, :, T - W:].contiguous(), "v_win": d["v"][:, :, T - W:].contiguous()}
    qbf = d["q"].contiguous()
    print(f"hybrid decode 32K batch 8 bench call, split {bench.HYBRID_SPLIT}", flush=True)
    out, lse = mxa.decode(qbf, kc, vc, d["ctx_len"], split_len=bench.HYBRID_SPLIT, hybrid=hy, return_lse=True)
    torch.cuda.synchronize()
    qd = oracle_dequant(*oracle_quantize(host_f64(d["q"][:, :, None, :]), "hd"), "hd")[:, :, 0]
    worst = 0.0
    for b, kv in picks:
        kd, vd = _oracle_kv(d["k"], d["v"], b, kv)
        toks = np.concatenate([oracle_sets[(b, kv)], np.arange(T - W, T)])
        kb, vb = host_f64(d["k"][b, kv]), host_f64(d["v"][b, kv])
        sets = {(0, 0): {"tokens": toks, "k": kb[toks], "v": vb[toks]}}
        ref = attention.decode(qd[b:b + 1, 4 * kv:4 * kv + 4], kd, vd, [T],
                               hybrid={"sets": sets, "q": host_f64(d["q"][b:b + 1, 4 * kv:4 * kv + 4])})
        worst = max(worst, _compare_group(out, lse, ref, b, kv, 4, "hybrid decode bench call"))
    print(f"  worst |err| {worst:.3e} over 12 pairs", flush=True)
