"""Benchmark of the MXFP4 attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Prints ONE JSON line.  The headline step is the 4K causal GQA prefill
(batch 1, 32 query / 8 KV heads, seq 4096, head_dim 128, bf16 inputs with
outlier K channels, static Smooth-QK): MXFP4 quantisation of Q, K, V plus the
attention kernel.  `value` is algorithmic TFLOP/s of that step (4*D flops per
unmasked query-key pair, the two contractions only).  The 32K decode legs
(plain and hybrid) are reported in the same line under "decode" and
"hybrid_decode" with ms/token, GB/s and their HBM roofline; the 32K
non-causal prefill with UOS scales (24 heads, 13.2 TFLOP per call) under
"diffusion_prefill" with its MXFP4 roofline.

Inputs are generated on the GPU from fixed seeds (synth); they are resident in
HBM before any timed region.  Calibration of the Smooth-QK factors is offline
(calibration-static) and not timed.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP4_TFLOPS = 10100.0   # MI355X dense MXFP4 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "MXFP4 attn prefill TFLOP/s; 32K decode ms/token + HBM GB/s (% roofline)"

# Launch configurations the legs time (tests/test_gpu_bench_configs.py runs
# the same calls against the oracle).
KV_TILE = 128           # prefill key tile
DECODE_SPLIT = 16384    # tokens per split, 32K batch-32 decode: 2 x 256 (sequence, KV head) = 512
                        # workgroups, one round at two per CU
HYBRID_SPLIT = 2752     # tokens per split, 32K batch-8 hybrid decode: 12 splits x 64 (sequence, KV head)
                        # = 768 workgroups, one round at three per CU
HYBRID_WINDOW = 128     # bf16 recent window (decode and hybrid prefill)

# HBM bytes per launch of the dominant kernels, from two rocprofv3 --pmc runs
# (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch) each scaled by what the same
# counter reads for an elementwise kernel of known size (--calibrate-copy).
# A figure is reported only while the kernel's sources hash to the profiled
# state; after any change to them it is null until profiled again.
PROFILED_TRAFFIC = {
    # 4K causal GQA step: fetch 6841.09 KiB x 2.000 + write 65572.91 KiB x 1.000 per dispatch (medians)
    "prefill_kernel<128,128,true,true>": {"bytes": 81157216, "sources": "01d8c7ff8dd1bf2f"},
    # 32K non-causal UOS (24 heads): fetch 429522.97 KiB x 2 + write 393216.0 KiB (median of 8); each XCD
    # runs one head's query blocks after another, whose K/V (4.46 MB) slightly exceed its 4 MB L2
    "prefill_kernel<128,128,false,true> uos": {"bytes": 1282316224, "sources": "01d8c7ff8dd1bf2f"},
    # 32K batch-32 call (bf16 query encoded in the scan): scan fetch 557328.2 KiB x 2 + write 1088 KiB
    # (median of 8), plus the merge (fetch 598.5 KiB x 2 + write 512 KiB)
    "decode_scan_kernel<128> split 16384": {"bytes": 1144272192, "sources": "beacda9caff5c1c1"},
    # 32K batch-8 hybrid call: scan fetch 168693.8 KiB x 2 + write 2176.5 KiB (median of 8) + merge
    # 2307072; the 4-bit rows of the bf16-held tokens are not fetched, but their 128-byte lines mostly
    # hold a neighbour that is
    "decode_scan_kernel<128> hybrid split 2752": {"bytes": 350020688, "sources": "beacda9caff5c1c1"},
}
TRAFFIC_SOURCES = {
    "prefill": ["bit_microscaled_flashattention_amd/csrc/prefill.hip",
                "bit_microscaled_flashattention_amd/csrc/mx_device.h",
                "bit_microscaled_flashattention_amd/csrc/kernels.h"],
    "decode": ["bit_microscaled_flashattention_amd/csrc/decode.hip",
               "bit_microscaled_flashattention_amd/csrc/mx_device.h",
               "bit_microscaled_flashattention_amd/csrc/kernels.h"],
}


def sources_digest(kind):
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES[kind]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def profiled_traffic(kind, key):
    """Profiled HBM bytes per launch of `key`, or None if absent or stale."""
    rec = PROFILED_TRAFFIC.get(key)
    if rec is None or rec["sources"] != sources_digest(kind):
        return None
    return rec["bytes"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--legs", default="prefill,diffusion,decode,hybrid,tiny",
                    help="comma list of legs to run (prefill is the headline); 'quant' (alone or with "
                         "other non-prefill legs) launches the 4K step's quantiser jobs one at a time")
    ap.add_argument("--kv-tile", type=int, default=KV_TILE)
    ap.add_argument("--decode-split", type=int, default=DECODE_SPLIT, help="tokens per split, 32K decode leg")
    ap.add_argument("--hybrid-split", type=int, default=HYBRID_SPLIT, help="tokens per split, hybrid decode leg")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run an elementwise kernel of known size (1 GiB in, 1 GiB out) three times, "
                         "to scale HBM byte counters; prints the source digests of the profiled kernels")
    return ap.parse_args()


def timed(fn, steps, warmup, kernel_fn=None):
    """Wall time per step over `steps` steps after `warmup` untimed ones, and
    the mean duration of kernel_fn: `steps` back-to-back launches bracketed
    by two events on the launch stream (the library launches on torch's
    current stream), total / steps.  Per-launch event pairs would add the
    host's call time whenever the queue runs dry."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    kern = None
    if kernel_fn is not None:
        kernel_fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            kernel_fn()
        b.record()
        torch.cuda.synchronize()
        kern = a.elapsed_time(b) / steps / 1e3
    return wall, kern


# Untimed load before the first timed leg.  The GPU raises its clocks only
# under sustained load: on these boxes the 4K prefill kernel takes 90-97 us
# in the first 20 ms after idle and 81-82 us from about 50 ms on.  The per-leg
# warmup steps stay as given; this settles the clocks once beforehand.
CLOCK_SETTLE_S = 0.15


def settle_clocks(fn, seconds=CLOCK_SETTLE_S):
    """Run fn repeatedly, untimed, for at least `seconds` of wall time."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while True:
        for _ in range(8):
            fn()
        n += 8
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return n


def launch_events(kernel_fn, n):
    """Durations of n launches of kernel_fn, each between its own two events
    on the launch stream, all enqueued before one synchronise so the queue
    runs ahead of the GPU.  Returns (mean, median) in seconds."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    kernel_fn()
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        kernel_fn()
        b.record()
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) / 1e3 for a, b in ev)
    return sum(ts) / n, ts[n // 2]


# ------------------------------------------------------------------ prefill
def quant_jobs_leg(args):
    """The 4K step's three quantiser jobs one at a time (Q and K in head-dim
    blocks with their Smooth-QK factors, V in key blocks), `steps` launches of
    each in that order, for per-job counter and trace runs."""
    import torch
    import bit_microscaled_flashattention_amd as mxa
    import synth

    B, HQ, HKV, S, D = 1, 32, 8, 4096, 128
    d = synth.gqa_prefill(device="cuda")
    qs, ks = mxa.smooth_calibrate(d["q_cal"], d["k_cal"])
    jobs = {"q_hd": dict(x=d["q"], chan_scale=qs, out=mxa.empty_mx((B, HQ, S, D), "hd")),
            "k_hd": dict(x=d["k"], chan_scale=ks, out=mxa.empty_mx((B, HKV, S, D), "hd")),
            "v_key": dict(x=d["v"], layout="key", out=mxa.empty_mx((B, HKV, S, D), "key"))}
    settle_clocks(lambda: mxa.quantize_batch(list(jobs.values())))
    res = {}
    for name, job in jobs.items():
        _, t = timed(lambda: None, args.steps, 0, lambda job=job: mxa.quantize_batch([job]))
        res[name] = {"ms": round(t * 1e3, 4)}
    res["note"] = ("the 4K step's quantiser jobs launched alone, in this order; ms is the back-to-back "
                   "launch time including the binding's per-call cost")
    return res


def prefill_leg(args):
    import torch
    import bit_microscaled_flashattention_amd as mxa
    import synth

    B, HQ, HKV, S, D = 1, 32, 8, 4096, 128
    d = synth.gqa_prefill(device="cuda")
    qs, ks = mxa.smooth_calibrate(d["q_cal"], d["k_cal"])        # offline, untimed
    qh = mxa.empty_mx((B, HQ, S, D), "hd")
    kh = mxa.empty_mx((B, HKV, S, D), "hd")
    vh = mxa.empty_mx((B, HKV, S, D), "key")
    out = torch.empty((B, HQ, S, D), dtype=torch.float32, device="cuda")

    def attn():
        mxa.prefill(qh, kh, vh, causal=True, kv_tile=args.kv_tile, out=out)

    # Q, K (with their Smooth-QK factors) and V quantised by one launch.
    qkv_jobs = [dict(x=d["q"], chan_scale=qs, out=qh), dict(x=d["k"], chan_scale=ks, out=kh),
                dict(x=d["v"], layout="key", out=vh)]

    def step():
        mxa.quantize_batch(qkv_jobs)
        attn()

    # The same step with Q and K rotated by the Walsh-Hadamard transform inside
    # the quantiser; the attention kernel is unchanged.
    rot_jobs = [dict(j, hadamard=True) if j.get("layout", "hd") == "hd" else j for j in qkv_jobs]

    def step_rot():
        mxa.quantize_batch(rot_jobs)
        attn()

    settle_clocks(step)
    wall, kern_b2b = timed(step, args.steps, args.warmup, attn)
    kern, kern_med = launch_events(attn, args.steps)
    # The same kernel writing bf16 outputs (half the output bytes).
    out_bf = torch.empty((B, HQ, S, D), dtype=torch.bfloat16, device="cuda")

    def attn_bf():
        mxa.prefill(qh, kh, vh, causal=True, kv_tile=args.kv_tile, out=out_bf)

    kern_bf, kern_bf_med = launch_events(attn_bf, args.steps)
    _, quant = timed(lambda: None, args.steps, 0, lambda: mxa.quantize_batch(qkv_jobs))
    wall_r, quant_r = timed(step_rot, args.steps, args.warmup, lambda: mxa.quantize_batch(rot_jobs))
    # Hybrid prefill: the top 5% vertical-line keys by column mass of the last
    # 64 queries, and a 128-key window per row, in bf16 (selection untimed
    # here, timed on its own).
    W = HYBRID_WINDOW
    ctx = torch.tensor([S], dtype=torch.int32, device="cuda")
    col = torch.zeros((B, HKV, S), dtype=torch.float32, device="cuda")
    # The last 64 queries with the same Smooth-QK factor as Q, against the
    # smoothed K the step wrote: their logits are those of the attention.
    qr = mxa.quantize(d["q"][:, :, S - 64:], "hd", chan_scale=qs)
    step()
    sel_ws = torch.empty(mxa.select_workspace_bytes(B, HQ, 64, S), dtype=torch.uint8, device="cuda")

    def select():
        col.zero_()
        return mxa.select_vertical(qr, kh, ctx, col, window=W, workspace=sel_ws)

    idx, nsel = select()

    def attn_h():
        mxa.prefill_hybrid(qh, kh, vh, d["q"], d["k"], d["v"], W, idx, nsel, kv_tile=args.kv_tile, out=out)

    def step_h():
        mxa.quantize_batch(qkv_jobs)
        attn_h()

    wall_h, kern_h = timed(step_h, args.steps, args.warmup, attn_h)
    _, sel_t = timed(lambda: None, args.steps, 0, select)
    # The plain step's output on the heads the CPU oracle later recomputes,
    # for the full-size comparison reported beside the oracle's time.  Taken
    # after all timing: the host copy idles the GPU, and its clocks drop.
    step()
    out_sample = out[:, list(range(0, HQ, 3))].cpu()
    pairs = B * HQ * S * (S + 1) // 2
    flops = 4 * D * pairs
    res = {
        "flops": flops, "step_s": wall, "kernel_s": kern, "kernel_median_s": kern_med, "kernel_b2b_s": kern_b2b,
        "step_tflops": flops / wall / 1e12, "kernel_tflops": flops / kern / 1e12,
        "quantize_s": quant, "out_sample": out_sample,
        "bf16_out": {"kernel_ms": round(kern_bf * 1e3, 4), "kernel_median_ms": round(kern_bf_med * 1e3, 4),
                     "kernel_tflops": round(flops / kern_bf / 1e12, 2),
                     "frac": round(flops / kern_bf / 1e12 / PEAK_FP4_TFLOPS, 4),
                     "note": "the same attention kernel writing bf16 instead of fp32 outputs"},
        "hybrid_prefill": {"ms_per_step": round(wall_h * 1e3, 4), "kernel_ms": round(kern_h * 1e3, 4),
                           "kernel_tflops": round(flops / kern_h / 1e12, 2),
                           "selection_ms": round(sel_t * 1e3, 4),
                           "n_sel_per_kv_head": int(nsel.max().item()), "window": W,
                           "note": "vertical-line keys (top 5% column mass of the last 64 queries over the "
                                   "non-window prefix) and a 128-key sliding window per row in bf16 under the "
                                   "same softmax; flops counted as for the 4-bit step"},
        "hadamard_qk": {"ms_per_step": round(wall_r * 1e3, 4), "step_tflops": round(flops / wall_r / 1e12, 2),
                        "quantize_ms": round(quant_r * 1e3, 4), "plain_quantize_ms": round(quant * 1e3, 4),
                        "note": "Q and K rows rotated by the normalised Walsh-Hadamard transform before MXFP4 "
                                "(in the quantiser launch); same attention kernel"},
    }
    return res, d, (qs, ks)


# ------------------------------------------------------------------ oracle timings
# The CPU oracle as it stands (float64 numpy, oracle/), timed on this host on a
# bounded seeded sample of each workload and scaled to the full one.  Query
# rows are independent, so the cost of a workload is a per-row part times its
# rows plus a per-head (or per KV head) part times its heads; both parts are
# measured and both the measured and the scaled seconds are reported.
def host_cores():
    """Threads the oracle may use: BLAS threads (numpy matmul); the
    elementwise numpy work is single-threaded.  Also the host's counts."""
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = os.cpu_count() or 1
    aff = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None
    return int(blas), {"os_cpu_count": os.cpu_count(), "affinity": aff, "blas_threads": int(blas)}


def _host(t):
    import torch
    return t.detach().to("cpu").to(torch.float64).numpy()


def prefill_cpu_baseline(d, cal, gpu_out=None):
    """The oracle on 11 of the 32 query heads (every third head), every row:
    quantisation of those heads' Q, K, V plus the tiled prefill with its
    rounding envelope.  Rate scaled to the full workload by the fraction of
    query-key pairs.  The same run records the per-tile mass change of P
    quantisation (HiFA4's tile diagnostic): eps = sum P_hat / sum P_tilde - 1
    per (query row, 128-key tile), and, given the GPU step's output on those
    heads, compares every row: |gpu - oracle| <= 2e-3 + envelope."""
    import numpy as np
    from oracle import attention, mx, smooth

    cores, info = host_cores()
    qs, ks = (c.cpu().numpy() for c in cal)
    heads = list(range(0, 32, 3))
    q = _host(d["q"][:, heads]).astype(np.float32)
    k = _host(d["k"]).astype(np.float32)
    v = _host(d["v"])
    S, D = q.shape[2], q.shape[3]
    eps = []
    par = {"rows": 0, "max_abs_err": 0.0, "rows_with_envelope": 0, "rows_over_bar": 0}
    t0 = time.perf_counter()
    pairs = 0
    for i, h in enumerate(heads):
        kv = h // 4
        q32 = smooth.apply(q[:, i:i + 1], qs[h:h + 1]).astype(np.float64)
        k32 = smooth.apply(k[:, kv:kv + 1], ks[kv:kv + 1]).astype(np.float64)
        qc, qsb = mx.quantize(q32, axis=3)
        kc, ksb = mx.quantize(k32, axis=3)
        vc, vsb = mx.quantize(v[:, kv:kv + 1], axis=2)
        res = attention.prefill_head(mx.dequantize(qc, qsb, 3)[0, 0], mx.dequantize(kc, ksb, 3)[0, 0],
                                     mx.dequantize(vc, vsb, 2)[0, 0], causal=True, kv_tile=KV_TILE,
                                     envelope=True, return_tile_eps=True)
        e = res["tile_eps"]
        eps.append(e[np.isfinite(e)])
        pairs += S * (S + 1) // 2
        if gpu_out is not None:
            err = np.abs(gpu_out[0, i].numpy().astype(np.float64) - res["out"]).max(axis=1)
            bnd = res["bound"]
            par["max_abs_err"] = max(par["max_abs_err"], float(err.max()))
            par["rows_with_envelope"] += int((bnd > 0).sum())
            par["rows_over_bar"] += int((err > 2e-3 + bnd).sum())
            par["rows"] += int(err.size)
    dt = time.perf_counter() - t0
    eps = np.concatenate(eps)
    out = {"value": 4 * D * pairs / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
           "sample": f"{len(heads)} of 32 query heads, all 4096 rows (quantise + tiled PNQ prefill, float64 "
                     f"numpy); {dt:.1f} s measured; rate scaled by pair count to the full workload",
           "seconds": round(dt, 2), "host": info}
    tile = {"eps_median": float(np.median(eps)), "eps_mean": float(eps.mean()),
            "eps_p10": float(np.percentile(eps, 10)), "eps_p90": float(np.percentile(eps, 90)),
            "tiles": int(eps.size),
            "note": "per (query row, 128-key tile): sum P_hat / sum P_tilde - 1 under OCP P scales, oracle, "
                    "the 11 sampled heads of the 4K step"}
    if gpu_out is not None:
        par["note"] = ("the timed step's fp32 output against the oracle on the same 11 heads, every row: "
                       "max |gpu - oracle| per row against 2e-3 + the oracle's rounding envelope")
        out["parity"] = par
    return out, tile


def tiny_cpu_oracle(d):
    """The whole tiny workload (quantise Q, K, V, one-tile PNQ prefill) on one
    BLAS thread and on all of them; repeated for at least 1 s each."""
    import numpy as np
    from oracle import attention, mx
    from threadpoolctl import threadpool_limits

    q, k, v = _host(d["q"]), _host(d["k"]), _host(d["v"])

    def run():
        qc, qsb = mx.quantize(q, axis=3)
        kc, ksb = mx.quantize(k, axis=3)
        vc, vsb = mx.quantize(v, axis=2)
        attention.prefill_head(mx.dequantize(qc, qsb, 3)[0, 0], mx.dequantize(kc, ksb, 3)[0, 0],
                               mx.dequantize(vc, vsb, 2)[0, 0], causal=False, kv_tile=KV_TILE)

    res = {}
    cores, info = host_cores()
    for label, n in (("1_core", 1), ("all_cores", cores)):
        with threadpool_limits(limits=n):
            run()
            reps, t0 = 0, time.perf_counter()
            while True:
                run()
                reps += 1
                if time.perf_counter() - t0 >= 1.0:
                    break
            res[label] = {"ms_per_step": round((time.perf_counter() - t0) / reps * 1e3, 3), "cores": n}
    res.update(kind="oracle", host=info,
               sample="the whole workload (1 x 1 x 128 x 64, fp16): quantise Q, K, V + one-tile PNQ prefill")
    return res


def decode_cpu_oracle(k_rows, v_rows, q_rows, n_seq, hq, hkv, tokens, alg_bytes, hybrid_sets=None, q_bf=None):
    """The oracle's decode step on seeded (sequence, query head) pairs:
    dequantise the MXFP4 cache rows of each pair's KV head (the cache is
    stored encoded; encoding it is not part of a step), encode the query,
    softmax over the context (plus the bf16 set when hybrid).

    k_rows/v_rows: {(b, kv): float64 [T, D] values the cache was encoded
    from}; q_rows: {(b, h): float64 [D]}.  Scaled as n_seq*hkv KV heads of
    dequantisation plus n_seq*hq pairs of attention."""
    import numpy as np
    from oracle import attention, mx

    cores, info = host_cores()
    g = hq // hkv
    cache = {key: (mx.quantize(k_rows[key], axis=1), mx.quantize(v_rows[key], axis=1)) for key in k_rows}
    t_deq, t_att = 0.0, 0.0
    for (b, kv), ((kc, ks), (vc, vs)) in cache.items():
        t0 = time.perf_counter()
        kd, vd = mx.dequantize(kc, ks, 1), mx.dequantize(vc, vs, 1)
        t1 = time.perf_counter()
        for h in range(kv * g, kv * g + g):
            if (b, h) not in q_rows:
                continue
            qc, qsb = mx.quantize(q_rows[(b, h)], axis=0)
            hy = None
            if hybrid_sets is not None:
                toks, kb, vb = hybrid_sets[(b, kv)]
                hy = {"tokens": toks, "k": kb, "v": vb, "q": q_bf[(b, h)]}
            attention.decode_head(mx.dequantize(qc, qsb, 0), kd, vd, tokens, hybrid=hy)
        t_deq += t1 - t0
        t_att += time.perf_counter() - t1
    n_kv, n_pairs = len(cache), len(q_rows)
    full = n_seq * hkv * t_deq / n_kv + n_seq * hq * t_att / n_pairs
    return {"value": round(full * 1e3, 2), "unit": "ms/token", "GB_per_s": round(alg_bytes / full / 1e9, 3),
            "cores": cores, "kind": "oracle", "host": info,
            "sample": f"{n_pairs} seeded (sequence, query head) pairs over {n_kv} KV heads: dequantise their "
                      f"cache rows, encode the query, {'hybrid ' if hybrid_sets else ''}softmax over {tokens} "
                      f"tokens; {t_deq + t_att:.2f} s measured, scaled to {n_seq * hkv} KV heads and "
                      f"{n_seq * hq} pairs",
            "measured_s": round(t_deq + t_att, 3), "scaled_s": round(full, 2)}


def diffusion_cpu_oracle(q, k, v, heads, rows):
    """The oracle on `rows` seeded query rows of each of `heads` (UOS on Q,
    K, V and P): encode the head's K and V and the sampled Q rows, tiled PNQ
    prefill of those rows.  Scaled to 24 heads x 32768 rows."""
    import numpy as np
    from oracle import attention, mx

    cores, info = host_cores()
    R = mx.RULE_UOS
    t_kv, t_q, t_att = 0.0, 0.0, 0.0
    S = k.shape[2]
    for i, h in enumerate(heads):
        t0 = time.perf_counter()
        kc, ksb = mx.quantize(k[:, i:i + 1], axis=3, rule=R)
        vc, vsb = mx.quantize(v[:, i:i + 1], axis=2, rule=R)
        kd, vd = mx.dequantize(kc, ksb, 3)[0, 0], mx.dequantize(vc, vsb, 2)[0, 0]
        t1 = time.perf_counter()
        qc, qsb = mx.quantize(q[:, i:i + 1], axis=3, rule=R)
        qd = np.zeros((S, q.shape[3]))
        qd[rows[i]] = mx.dequantize(qc, qsb, 3)[0, 0]
        t2 = time.perf_counter()
        attention.prefill_head(qd, kd, vd, causal=False, kv_tile=KV_TILE, p_rule=R, rows=rows[i])
        t_kv += t1 - t0
        t_q += t2 - t1
        t_att += time.perf_counter() - t2
    n_rows = sum(len(r) for r in rows)
    full = 24 * t_kv / len(heads) + 24 * S * (t_q + t_att) / n_rows
    flops = 4 * 128 * 24 * S * S
    return {"value": flops / full / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle", "host": info,
            "sample": f"{len(rows[0])} seeded rows of each of {len(heads)} heads (encode K, V and the rows, tiled "
                      f"PNQ prefill, UOS); {t_kv + t_q + t_att:.1f} s measured, scaled to 24 heads x {S} rows",
            "measured_s": round(t_kv + t_q + t_att, 2), "scaled_s": round(full, 1)}


# ------------------------------------------------------------------ decode
def _flush_buffer():
    import torch
    return torch.ones(512 << 20, dtype=torch.uint8, device="cuda")


def timed_flushed(fn, steps, warmup, flush):
    """Mean duration of fn over `steps` calls, each timed with events on the
    current stream, with a read of an unrelated 512 MB buffer between calls
    (not timed) so the 256 MB Infinity Cache holds none of the previous step's
    bytes.  The flush reads rather than writes: written lines would be dirty
    and their write-back would land inside the next timed call."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    total = 0.0
    for i in range(steps):
        flush.view(torch.int32).sum()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        total += a.elapsed_time(b) / 1e3
    return total / steps


def decode_leg(args, flush):
    import torch
    import bit_microscaled_flashattention_amd as mxa
    import synth

    B, HQ, HKV, T, D = 32, 32, 8, 32768, 128
    SPLIT = args.decode_split
    d = synth.long_decode(device="cuda")
    kc, vc = mxa.quantize(d["k"], "hd"), mxa.quantize(d["v"], "hd")
    # Host copies for the oracle's timing sample: four seeded (sequence, query
    # head) pairs over two KV heads.
    picks = [(5, 1), (26, 6)]
    cpu_pairs = [(5, 4), (5, 6), (26, 25), (26, 27)]
    k_rows = {key: _host(d["k"][key]) for key in picks} if args.cpu else None
    v_rows = {key: _host(d["v"][key]) for key in picks} if args.cpu else None
    q_rows = {key: _host(d["q"][key]) for key in cpu_pairs} if args.cpu else None
    del d["k"], d["v"]
    torch.cuda.empty_cache()
    qh = mxa.empty_mx((B, HQ, 1, D), "hd")
    ws = torch.empty(mxa.decode_workspace_bytes(B, HQ, HKV, D, T, SPLIT), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, HQ, D), dtype=torch.float32, device="cuda")
    q4 = d["q"][:, :, None, :]

    qbf = d["q"].contiguous()

    # One call per token: the scan encodes the bf16 query itself.
    def call():
        mxa.decode(qbf, kc, vc, d["ctx_len"], split_len=SPLIT, workspace=ws, out=out)

    # The same step as two launches: the quantiser, then the scan on its codes.
    def step_two_launches():
        mxa.quantize(q4, "hd", out=qh)
        mxa.decode(qh, kc, vc, d["ctx_len"], split_len=SPLIT, workspace=ws, out=out)

    # The same decode with a dual-residual query (two MXFP4 query halves,
    # one more QK^T MFMA per chunk).
    q1 = mxa.empty_mx((B, HQ, 1, D), "hd")
    q2 = mxa.empty_mx((B, HQ, 1, D), "hd")

    def call_dual():
        mxa.decode(q1, kc, vc, d["ctx_len"], split_len=SPLIT, workspace=ws, out=out, q_res=q2)

    def step_dual():
        mxa.quantize_dual(q4, out=q1, out_res=q2)
        call_dual()

    t_call = timed_flushed(call, args.steps, args.warmup, flush)
    t_step = t_call
    t_step2 = timed_flushed(step_two_launches, args.steps, args.warmup, flush)
    t_call_d = timed_flushed(call_dual, args.steps, args.warmup, flush)
    t_step_d = timed_flushed(step_dual, args.steps, args.warmup, flush)

    # The same cache as a shuffled pool of 64-token pages behind a block table.
    PAGE = 64
    maxp = T // PAGE
    perm = torch.randperm(B * maxp, generator=torch.Generator().manual_seed(7))
    table = perm.reshape(B, maxp).to(torch.int32).contiguous().cuda()

    def to_pool(c):
        def scatter(x):
            src = x.reshape(B, HKV, maxp, PAGE, x.shape[-1]).permute(0, 2, 1, 3, 4).reshape(B * maxp, HKV, PAGE, -1)
            dst = torch.empty_like(src)
            dst[perm.cuda()] = src
            return dst
        return mxa.MX(scatter(c.codes), scatter(c.scales), (B * maxp, HKV, PAGE, D), "hd")

    kp = to_pool(kc)
    del kc
    vp = to_pool(vc)
    del vc
    torch.cuda.empty_cache()

    # A split spans at most 64 pages.
    split_p = min(SPLIT, 64 * PAGE)
    ws_p = torch.empty(mxa.decode_workspace_bytes(B, HQ, HKV, D, T, split_p), dtype=torch.uint8, device="cuda")

    def call_paged():
        mxa.decode_paged(qbf, kp, vp, table, d["ctx_len"], split_len=split_p, workspace=ws_p, out=out)

    t_call_p = timed_flushed(call_paged, args.steps, args.warmup, flush)
    cache_bytes = B * HKV * T * (D // 2 + D // 32) * 2
    # The one-call step reads the bf16 query (the scan encodes it); the dual
    # call reads both encoded halves.
    q_bytes = B * HQ * D * 2
    q_mx_bytes = B * HQ * (D // 2 + D // 32)
    alg = cache_bytes + q_bytes + B * HQ * D * 4
    alg_d = cache_bytes + 2 * q_mx_bytes + B * HQ * D * 4
    cpu = decode_cpu_oracle(k_rows, v_rows, q_rows, B, HQ, HKV, T, alg) if args.cpu else None
    return {
        "workload": "batch 32, 32/8 heads, head_dim 128, ctx 32768, MXFP4 K/V cache (E2M1 + E8M0 per 32 "
                    f"along head_dim), MXFP4 query, split {SPLIT}; step = one decode call (the scan encodes the "
                    "bf16 query, then the merge)",
        "ms_per_token": round(t_step * 1e3, 4),
        "ms_per_token_two_launches": round(t_step2 * 1e3, 4),
        "GB_per_s": round(alg / t_step / 1e9, 1),
        "algorithmic_bytes": alg,
        "roofline": {"bound": "hbm", "kernel": "mxattn_decode (decode_scan_kernel<128> + merge)",
                     "achieved": round(alg / t_call / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(alg / t_call / 1e9 / PEAK_HBM_GBS, 4),
                     "call_ms": round(t_call * 1e3, 4),
                     "traffic": profiled_traffic("decode", f"decode_scan_kernel<128> split {SPLIT}")},
        "cache": "flushed (512 MB read of another buffer) before every timed step",
        "dual_residual_query": {
            "ms_per_token": round(t_step_d * 1e3, 4),
            "call_ms": round(t_call_d * 1e3, 4),
            "achieved_GB_per_s": round(alg_d / t_call_d / 1e9, 1),
            "frac": round(alg_d / t_call_d / 1e9 / PEAK_HBM_GBS, 4),
            "note": "q split into MXFP4(q) + MXFP4(q - dequant(MXFP4(q))); step = quantise both halves + decode",
        },
        "cpu_oracle": cpu,
        "paged_kv": {
            "call_ms": round(t_call_p * 1e3, 4),
            "achieved_GB_per_s": round(alg / t_call_p / 1e9, 1),
            "frac": round(alg / t_call_p / 1e9 / PEAK_HBM_GBS, 4),
            "note": f"same cache as a shuffled pool of {PAGE}-token pages (block table [32, {maxp}]), split {split_p}",
        },
    }


def hybrid_leg(args, flush):
    import torch
    import bit_microscaled_flashattention_amd as mxa
    import synth

    B, HQ, HKV, T, D, W = 8, 32, 8, 32768, 128, HYBRID_WINDOW
    SPLIT = args.hybrid_split
    d = synth.hybrid_decode(device="cuda")
    kc, vc = mxa.quantize(d["k"], "hd"), mxa.quantize(d["v"], "hd")
    qr = mxa.quantize(d["q_recent"], "hd")
    col = torch.zeros((B, HKV, T), dtype=torch.float32, device="cuda")
    sel_ws = torch.empty(mxa.select_workspace_bytes(B, HQ, 64, T), dtype=torch.uint8, device="cuda")

    def select():
        return mxa.select_vertical(qr, kc, d["ctx_len"], col, window=W, workspace=sel_ws)

    idx, n = select()
    cpu = None
    if args.cpu:
        cpu = hybrid_cpu_oracle(d, [(1, 2), (6, 5)], [(1, 8), (1, 11), (6, 20), (6, 22)], T, W)
    # Gather the bf16 rows of the selected tokens (the method keeps them in
    # full precision), timed with the selection it follows.
    max_sel = idx.shape[-1]
    k_sel = torch.empty((B, HKV, max_sel, D), dtype=torch.bfloat16, device="cuda")
    v_sel = torch.empty_like(k_sel)

    def gather():
        mxa.gather_rows(d["k"], d["v"], idx, n, k_sel, v_sel)

    gather()
    hy = {"idx": idx, "n_sel": n, "window": W, "k_sel": k_sel, "v_sel": v_sel,
          "k_win": d["k"][:, :, T - W:].contiguous(), "v_win": d["v"][:, :, T - W:].contiguous()}
    qh = mxa.empty_mx((B, HQ, 1, D), "hd")
    ws = torch.empty(mxa.decode_workspace_bytes(B, HQ, HKV, D, T, SPLIT, max_sel + W), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((B, HQ, D), dtype=torch.float32, device="cuda")
    q4 = d["q"][:, :, None, :]
    qbf = d["q"].contiguous()

    # One call per token: the scan encodes the bf16 query for the 4-bit tokens.
    def call():
        mxa.decode(qbf, kc, vc, d["ctx_len"], split_len=SPLIT, hybrid=hy, workspace=ws, out=out)

    def step_two_launches():
        mxa.quantize(q4, "hd", out=qh)
        mxa.decode(qh, kc, vc, d["ctx_len"], split_len=SPLIT, hybrid=hy, q_bf16=qbf, workspace=ws, out=out)

    t_call = timed_flushed(call, args.steps, args.warmup, flush)
    t_step = t_call
    t_step2 = timed_flushed(step_two_launches, args.steps, args.warmup, flush)
    t_sel = timed_flushed(select, max(args.steps // 4, 3), 1, flush)
    t_gather = timed_flushed(gather, max(args.steps // 4, 3), 1, flush)
    del d["k"], d["v"]
    torch.cuda.empty_cache()
    nsel = int(n[0, 0].item())
    n4 = T - W - nsel
    per_pair = n4 * (D // 2 + D // 32) * 2 + (nsel + W) * D * 2 * 2 + nsel * 4
    alg = B * HKV * per_pair + B * HQ * 2 * D + B * HQ * D * 4     # bf16 query read once per head
    return {
        "workload": "batch 8, 32/8 heads, head_dim 128, ctx 32768, heavy-tailed column bias; 1632 selected "
                    "(top 5% of the non-window prefix by column mass) + 128-token window in bf16, rest MXFP4, "
                    f"one softmax, split {SPLIT}; step = one hybrid decode call (the scan encodes the bf16 query)",
        "ms_per_token": round(t_step * 1e3, 4),
        "ms_per_token_two_launches": round(t_step2 * 1e3, 4),
        "GB_per_s": round(alg / t_step / 1e9, 1),
        "algorithmic_bytes": alg,
        "bf16_overhead_of_nonwindow_kv": round(nsel * (2 * D * 2 - (D // 2 + D // 32) * 2) /
                                               ((T - W) * (D // 2 + D // 32) * 2), 4),
        "selection_ms": round(t_sel * 1e3, 4),
        "gather_ms": round(t_gather * 1e3, 4),
        "selection_share_of_64_steps": round((t_sel + t_gather) / (t_sel + t_gather + 64 * t_step), 4),
        "selection_share_note": "(selection call + bf16 gather of the selected rows) / (that + 64 hybrid decode "
                                "calls): one refresh every 64 tokens",
        "roofline": {"bound": "hbm", "kernel": "mxattn_decode hybrid (one scan launch: fp4 splits + bf16 parts; merge)",
                     "achieved": round(alg / t_call / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(alg / t_call / 1e9 / PEAK_HBM_GBS, 4),
                     "call_ms": round(t_call * 1e3, 4),
                     "traffic": profiled_traffic("decode", f"decode_scan_kernel<128> hybrid split {SPLIT}")},
        "cache": "flushed (512 MB read of another buffer) before every timed step",
        "cpu_oracle": None if cpu is None else dict(cpu["decode"], GB_per_s=round(alg / cpu["decode_s"] / 1e9, 3)),
        "selection_cpu_oracle": None if cpu is None else cpu["selection"],
    }


def hybrid_cpu_oracle(d, picks, pairs, T, W):
    """The oracle's selection (encode the 64 recent queries of the KV head's
    four query heads and the keys, column mass, top 5%) on `picks` KV heads,
    then its hybrid decode step on `pairs` with those sets; both scaled to
    batch 8 x 8 KV heads (x 4 query heads)."""
    import numpy as np
    from oracle import mx, select

    cores, info = host_cores()
    k_rows = {key: _host(d["k"][key]) for key in picks}
    v_rows = {key: _host(d["v"][key]) for key in picks}
    sets, t_sel = {}, 0.0
    for (b, kv) in picks:
        qr = _host(d["q_recent"][b, 4 * kv:4 * kv + 4]).reshape(-1, k_rows[(b, kv)].shape[1])
        t0 = time.perf_counter()
        qc, qsb = mx.quantize(qr, axis=1)
        kc, ksb = mx.quantize(k_rows[(b, kv)], axis=1)
        cm = select.colmass_update(np.zeros(T), mx.dequantize(qc, qsb, 1), mx.dequantize(kc, ksb, 1), T)
        sel = select.topk_vertical(cm, T, W, 5, 100)
        t_sel += time.perf_counter() - t0
        toks = np.concatenate([sel, np.arange(T - W, T)])
        sets[(b, kv)] = (toks, k_rows[(b, kv)][toks], v_rows[(b, kv)][toks])
    q_rows = {key: _host(d["q"][key]) for key in pairs}
    dec = decode_cpu_oracle(k_rows, v_rows, q_rows, 8, 32, 8, T, 1, hybrid_sets=sets, q_bf=q_rows)
    dec.pop("GB_per_s")
    sel_full = 64 * t_sel / len(picks)
    return {"decode": dec, "decode_s": dec["scaled_s"],
            "selection": {"value": round(sel_full * 1e3, 1), "unit": "ms per selection call", "cores": cores,
                          "kind": "oracle", "host": info,
                          "sample": f"{len(picks)} KV heads: encode 256 recent queries and 32768 keys, column "
                                    f"mass, top 5%; {t_sel:.2f} s measured, scaled to 64 KV heads"}}


# ------------------------------------------------------------------ long non-causal
def diffusion_leg(args):
    """Non-causal video-diffusion-style prefill: batch 1, 24 heads, seq 32768
    (8 x 64 x 64 token grid), head_dim 128, low-rank spatially correlated
    bf16 Q/K/V; UOS (Qmax 7.25) scales on Q, K, V and P; P-Reordering/PNQ."""
    import torch
    import bit_microscaled_flashattention_amd as mxa
    import synth

    B, H, S, D = 1, 24, 32768, 128
    d = synth.diffusion(device="cuda")
    qh = mxa.empty_mx((B, H, S, D), "hd")
    kh = mxa.empty_mx((B, H, S, D), "hd")
    vh = mxa.empty_mx((B, H, S, D), "key")
    out = torch.empty((B, H, S, D), dtype=torch.float32, device="cuda")
    jobs = [dict(x=d["q"], rule="uos", out=qh), dict(x=d["k"], rule="uos", out=kh),
            dict(x=d["v"], layout="key", rule="uos", out=vh)]

    def attn():
        mxa.prefill(qh, kh, vh, causal=False, kv_tile=args.kv_tile, p_rule="uos", out=out)

    def step():
        mxa.quantize_batch(jobs)
        attn()

    steps, warm = max(args.steps // 4, 3), max(args.warmup // 2, 1)
    wall, _ = timed(step, steps, warm)
    kern, kern_med = launch_events(attn, steps)
    flops = 4 * D * B * H * S * S
    cpu = None
    if args.cpu:
        import numpy as np
        heads = [0, 13]
        rng = np.random.default_rng(5005)
        rows = [np.sort(rng.choice(S, size=256, replace=False)) for _ in heads]
        idx = [torch.as_tensor(r, device="cuda") for r in rows]
        qs = np.stack([_host(d["q"][0, h].index_select(0, ix)) for h, ix in zip(heads, idx)])[None]
        ks = _host(d["k"][:, heads])
        vs = _host(d["v"][:, heads])
        cpu = diffusion_cpu_oracle(qs, ks, vs, heads, rows)
    del d, out
    torch.cuda.empty_cache()
    return {
        "workload": "non-causal video-diffusion attention: batch 1, 24 heads, seq 32768 (8x64x64 grid), head_dim "
                    "128, bf16 Q/K/V with 16 low-frequency Fourier modes (lambda 0.5), UOS Qmax 7.25 on Q, K, V "
                    f"and P, PNQ, kv_tile {args.kv_tile}; step = quantise Q,K,V + attention",
        "ms_per_step": round(wall * 1e3, 4),
        "step_tflops": round(flops / wall / 1e12, 2),
        "flops": flops,
        "roofline": {"bound": "mfma", "kernel": "prefill_kernel<128,128,non-causal,uos>",
                     "achieved": round(flops / kern / 1e12, 2), "peak": PEAK_FP4_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(flops / kern / 1e12 / PEAK_FP4_TFLOPS, 4),
                     "kernel_ms": round(kern * 1e3, 4), "kernel_median_ms": round(kern_med * 1e3, 4),
                     "traffic": profiled_traffic("prefill", "prefill_kernel<128,128,false,true> uos")},
        "cpu_oracle": cpu,
    }


def tiny_leg(args):
    """The tiny workload (batch 1, one head, 128 x 64, fp16, non-causal, OCP):
    quantise Q, K, V + attention; launch-bound, no roofline claim."""
    import torch
    import bit_microscaled_flashattention_amd as mxa
    import synth

    d = synth.tiny(device="cuda")
    out = torch.empty((1, 1, 128, 64), dtype=torch.float32, device="cuda")
    qh, kh = mxa.empty_mx((1, 1, 128, 64), "hd"), mxa.empty_mx((1, 1, 128, 64), "hd")
    vh = mxa.empty_mx((1, 1, 128, 64), "key")
    jobs = [dict(x=d["q"], out=qh), dict(x=d["k"], out=kh), dict(x=d["v"], layout="key", out=vh)]

    def step():
        mxa.quantize_batch(jobs)
        mxa.prefill(qh, kh, vh, causal=False, kv_tile=KV_TILE, out=out)

    wall, _ = timed(step, args.steps, args.warmup)
    # The same step captured once as a HIP graph and replayed: the calls
    # allocate nothing when outputs are passed in, so the whole step replays
    # without the host-side launch path.
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    wall_g, _ = timed(graph.replay, args.steps, args.warmup)
    res = {"workload": "batch 1, 1 head, seq 128, head_dim 64, fp16 N(0,1), non-causal, OCP, one 128-key tile; "
                       "step = quantise Q, K, V (one launch) + attention",
           "ms_per_step": round(wall * 1e3, 4), "ms_per_step_graph": round(wall_g * 1e3, 4),
           "flops": 4 * 64 * 128 * 128,
           "note": "launch-bound: two launches of a few microseconds each; ms_per_step_graph replays the "
                   "step captured as one HIP graph"}
    if args.cpu:
        res["cpu_oracle"] = tiny_cpu_oracle(d)
    return res


def hbm_reference():
    """What torch's own kernels reach on this device, as context for the HBM
    fractions: a bf16 matrix-vector product over a 2 GiB matrix (a streaming
    read: the vendor BLAS kernel, the fastest read measured here), a sum over
    4 GiB (read) and a 2 GiB device copy (read+write)."""
    import torch
    res = {}
    a = torch.ones((1 << 20, 1024), dtype=torch.bfloat16, device="cuda")
    xv = torch.ones(1024, dtype=torch.bfloat16, device="cuda")
    settle_clocks(lambda: torch.mv(a, xv), 0.2)
    mean, med = launch_events(lambda: torch.mv(a, xv), 20)
    res["gemv_read_2GiB"] = {"GB_per_s": round((2 << 30) / med / 1e9, 1), "ms": round(med * 1e3, 3)}
    del a, xv
    x = torch.ones(1 << 30, dtype=torch.int32, device="cuda")
    y = torch.empty(1 << 29, dtype=torch.int32, device="cuda")
    for name, fn, nbytes in (("sum_read_4GiB", lambda: x.sum(), 4 << 30),
                             ("copy_2GiB", lambda: y.copy_(x[: 1 << 29]), 4 << 30)):
        mean, med = launch_events(fn, 5)
        res[name] = {"GB_per_s": round(nbytes / med / 1e9, 1), "ms": round(med * 1e3, 3)}
    del x, y
    torch.cuda.empty_cache()
    res["note"] = ("torch kernels, median of event-timed launches; bytes counted once each way; the matrix-vector "
                   "product is the practical read ceiling against which the decode scans' fractions can be read")
    return res


def main():
    args = parse()
    args.cpu = not args.no_cpu_baseline
    if args.gpus != 1:
        print("bench.py: the library runs on one GPU; --gpus must be 1 "
              "(multi-GPU sharding is a design note, not a measured path)", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.calibrate_copy:
        x = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            torch.neg(x, out=y)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "torch.neg int32", "bytes_read": x.numel() * 4,
                          "bytes_written": y.numel() * 4,
                          "sources": {k: sources_digest(k) for k in TRAFFIC_SOURCES}}))
        return
    legs = set(args.legs.split(","))

    def progress(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    if "prefill" not in legs:
        # Profiling runs of single legs: no headline figure.
        line = {"metric": METRIC, "value": None, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
                "warmup": args.warmup, "legs": sorted(legs)}
        flush = _flush_buffer()
        if "diffusion" in legs:
            line["diffusion_prefill"] = diffusion_leg(args)
            progress("diffusion leg done")
        if "decode" in legs:
            line["decode"] = decode_leg(args, flush)
            torch.cuda.empty_cache()
            progress("decode leg done")
        if "hybrid" in legs:
            line["hybrid_decode"] = hybrid_leg(args, flush)
            progress("hybrid leg done")
        if "tiny" in legs:
            line["tiny"] = tiny_leg(args)
        if "quant" in legs:
            line["quantize_jobs"] = quant_jobs_leg(args)
        print(json.dumps(line), flush=True)
        return
    pre, d, cal = prefill_leg(args)
    progress("prefill leg done")
    line = {
        "metric": METRIC,
        "value": round(pre["step_tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["step_s"] * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4",
        "data": "synthetic",
        "clock_settle_s": CLOCK_SETTLE_S,
        "clock_settle_note": "untimed prefill steps for this long before the first timed leg, so the GPU "
                             "clocks have left their idle state; then the warmup steps and the timed steps "
                             "as given",
        "config": {"workload": "causal GQA prefill: batch 1, 32 query / 8 KV heads, seq 4096, head_dim 128, "
                               "bf16 N(0,1) with 4 K channels x12 per KV head, static Smooth-QK, OCP scales, "
                               f"P-Reordering/PNQ, kv_tile {args.kv_tile}; step = quantise Q,K,V + attention",
                   "global_batch": 1, "seq_len": 4096, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "kernel": "prefill_kernel<128,128,causal,pnq>",
                     "achieved": round(pre["kernel_tflops"], 2), "peak": PEAK_FP4_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(pre["kernel_tflops"] / PEAK_FP4_TFLOPS, 4),
                     "kernel_ms": round(pre["kernel_s"] * 1e3, 4),
                     "kernel_median_ms": round(pre["kernel_median_s"] * 1e3, 4),
                     "kernel_back_to_back_ms": round(pre["kernel_b2b_s"] * 1e3, 4),
                     "timing": "kernel_ms: mean of per-launch event pairs on the launch stream, queue kept full; "
                               "back_to_back: two events around all launches / launches",
                     "traffic": profiled_traffic("prefill", "prefill_kernel<128,128,true,true>")},
        "bf16_out": pre["bf16_out"],
        "hadamard_qk": pre["hadamard_qk"],
        "hybrid_prefill": pre["hybrid_prefill"],
    }
    del d
    torch.cuda.empty_cache()
    if "diffusion" in legs:
        line["diffusion_prefill"] = diffusion_leg(args)
        progress("diffusion leg done")
    if legs & {"decode", "hybrid"}:
        flush = _flush_buffer()
        if "decode" in legs:
            line["decode"] = decode_leg(args, flush)
            torch.cuda.empty_cache()
            progress("decode leg done")
        if "hybrid" in legs:
            line["hybrid_decode"] = hybrid_leg(args, flush)
            torch.cuda.empty_cache()
            progress("hybrid leg done")
        del flush
    if "tiny" in legs:
        line["tiny"] = tiny_leg(args)
    line["hbm_reference"] = hbm_reference()
    if args.cpu:
        progress("timing the CPU oracle")
        d2 = __import__("synth").gqa_prefill(device="cuda")
        line["cpu_baseline"], line["tile_mass_loss"] = prefill_cpu_baseline(d2, cal, pre["out_sample"])
        del d2
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
