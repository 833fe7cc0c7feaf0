"""Seeded synthetic inputs for the five attention workloads.

This module draws random tensors and nothing else: it holds none of the
attention or quantisation arithmetic.  Both the HIP path (through the tests
and the benchmark) and the CPU oracle receive exactly these tensors.

Every tensor comes from its own ``torch.Generator`` seeded with
``1000 * stream + tensor_id``, where ``stream`` is a fixed id per generator
function (tiny 1, gqa_prefill 2, long_decode 3, hybrid_decode 4,
diffusion 5) and the tensor ids are Q 1, K 2, V 3, calibration 4,
structure 5, recent queries 6.  Values are drawn in float32 and rounded to
bfloat16/float16 by torch's round-to-nearest-even cast.  The numbers a
generator produces depend on the device it lives on, so a workload generated on the
GPU is copied back to the host before the oracle sees it (never regenerated
on the CPU).
"""

import math

import torch

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_CAL, TENSOR_STRUCT, TENSOR_RECENT = 1, 2, 3, 4, 5, 6


def seed_of(stream, tensor_id):
    return 1000 * int(stream) + int(tensor_id)


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def randn(shape, seed, device="cpu", dtype=torch.bfloat16, scale=1.0):
    g = _gen(device, seed)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if scale != 1.0:
        x = x * scale
    return x.to(dtype)


# ---------------------------------------- tiny non-causal prefill
def tiny(device="cpu", seq=128, head_dim=64, seed_base=1):
    """Batch 1, one head, fp16 Q/K/V ~ N(0, 1)."""
    shp = (1, 1, seq, head_dim)
    return {
        "q": randn(shp, seed_of(seed_base, TENSOR_Q), device, torch.float16),
        "k": randn(shp, seed_of(seed_base, TENSOR_K), device, torch.float16),
        "v": randn(shp, seed_of(seed_base, TENSOR_V), device, torch.float16),
    }


# ------------------------------------------ 4K causal GQA prefill
def gqa_prefill(device="cpu", batch=1, hq=32, hkv=8, seq=4096, head_dim=128,
                n_outlier=4, outlier_gain=12.0, cal_tokens=256, stream=2):
    """bf16 N(0,1) Q/K/V; per KV head ``n_outlier`` K channels (seeded choice
    without replacement) multiplied by ``outlier_gain``; a separate calibration
    slice of ``cal_tokens`` tokens drawn the same way."""
    gs = _gen("cpu", seed_of(stream, TENSOR_STRUCT))
    chans = torch.stack([torch.randperm(head_dim, generator=gs)[:n_outlier] for _ in range(hkv)])
    gain = torch.ones(hkv, head_dim)
    gain.scatter_(1, chans, outlier_gain)
    gain = gain.to(device)[None, :, None, :]

    def make_k(shape, seed):
        g = _gen(device, seed)
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        return (x * gain).to(torch.bfloat16)

    q = randn((batch, hq, seq, head_dim), seed_of(stream, TENSOR_Q), device)
    k = make_k((batch, hkv, seq, head_dim), seed_of(stream, TENSOR_K))
    v = randn((batch, hkv, seq, head_dim), seed_of(stream, TENSOR_V), device)
    gc = _gen(device, seed_of(stream, TENSOR_CAL))
    q_cal = torch.randn((hq, cal_tokens, head_dim), generator=gc, device=device).to(torch.bfloat16)
    k_cal = (torch.randn((1, hkv, cal_tokens, head_dim), generator=gc, device=device)
             * gain).to(torch.bfloat16)[0]
    return {"q": q, "k": k, "v": v, "q_cal": q_cal, "k_cal": k_cal, "outlier_channels": chans}


# ------------------------------------------- 32K decode, batch 32
def long_decode(device="cpu", batch=32, hq=32, hkv=8, ctx=32768, head_dim=128, stream=3):
    """bf16 N(0,1) keys/values for the cache and one N(0,1) query per head."""
    return {
        "q": randn((batch, hq, head_dim), seed_of(stream, TENSOR_Q), device),
        "k": randn((batch, hkv, ctx, head_dim), seed_of(stream, TENSOR_K), device),
        "v": randn((batch, hkv, ctx, head_dim), seed_of(stream, TENSOR_V), device),
        "ctx_len": torch.full((batch,), ctx, dtype=torch.int32, device=device),
    }


# ------------------------------------- 32K hybrid decode, batch 8
# Chosen so that the heaviest 5% of the non-window keys carry about 60% of the
# attention mass of the recent queries (mean over the KV heads; the HyQuant
# page reports 54-64% for real models).  Checked by tests/test_synth.py.
HYBRID_GAMMA = 0.19    # key offset gain along the bias direction
HYBRID_BETA = 1.0      # query offset along the bias direction
PARETO_SHAPE = 1.5


def hybrid_decode(device="cpu", batch=8, hq=32, hkv=8, ctx=32768, head_dim=128,
                  recent=64, gamma=HYBRID_GAMMA, beta=HYBRID_BETA, stream=4):
    """bf16 N(0,1) keys/values/queries with a heavy-tailed column bias.

    Per (batch, KV head) a seeded unit vector u; every key gets
    gamma * z_t * u with z_t ~ Pareto(shape 1.5) i.i.d. (inverse-CDF draw), and
    every query (current and recent) gets beta * u, so a few keys dominate the
    attention of all queries of that KV head, as vertical lines do.
    """
    gs = _gen(device, seed_of(stream, TENSOR_STRUCT))
    u = torch.randn((batch, hkv, head_dim), generator=gs, device=device)
    u = u / u.norm(dim=-1, keepdim=True)
    unif = torch.rand((batch, hkv, ctx), generator=gs, device=device)
    z = (1.0 - unif).clamp_min(1e-12).pow(-1.0 / PARETO_SHAPE)
    gk = _gen(device, seed_of(stream, TENSOR_K))
    k = torch.randn((batch, hkv, ctx, head_dim), generator=gk, device=device)
    k = (k + gamma * z[..., None] * u[:, :, None, :]).to(torch.bfloat16)
    del z, unif
    v = randn((batch, hkv, ctx, head_dim), seed_of(stream, TENSOR_V), device)
    g = hq // hkv
    ug = u.repeat_interleave(g, dim=1)                       # [B, Hq, D]
    gq = _gen(device, seed_of(stream, TENSOR_Q))
    q = (torch.randn((batch, hq, head_dim), generator=gq, device=device) + beta * ug)
    gr = _gen(device, seed_of(stream, TENSOR_RECENT))
    qr = (torch.randn((batch, hq, recent, head_dim), generator=gr, device=device)
          + beta * ug[:, :, None, :])
    return {
        "q": q.to(torch.bfloat16), "k": k, "v": v, "q_recent": qr.to(torch.bfloat16),
        "ctx_len": torch.full((batch,), ctx, dtype=torch.int32, device=device),
    }


# ---------------------------------------- video-diffusion prefill
def diffusion(device="cpu", batch=1, heads=24, frames=8, height=64, width=64,
              head_dim=128, n_modes=16, lam=0.5, stream=5):
    """bf16 Q/K/V = sqrt(1-lam) Z + sqrt(lam) F W: Z ~ N(0,1); tokens on a
    frames x height x width grid; F holds ``n_modes`` seeded low-frequency
    Fourier modes over the grid (unit variance); W ~ N(0, 1/n_modes) per head
    and per tensor."""
    seq = frames * height * width
    gs = _gen("cpu", seed_of(stream, TENSOR_STRUCT))
    ft = torch.randint(0, 3, (n_modes,), generator=gs).float()
    fh = torch.randint(0, 5, (n_modes,), generator=gs).float()
    fw = torch.randint(0, 5, (n_modes,), generator=gs).float()
    ph = torch.rand((n_modes,), generator=gs) * 2 * math.pi
    tt, hh, ww = torch.meshgrid(torch.arange(frames).float(), torch.arange(height).float(),
                                torch.arange(width).float(), indexing="ij")
    arg = (2 * math.pi * (tt.reshape(-1, 1) * ft / frames + hh.reshape(-1, 1) * fh / height
                          + ww.reshape(-1, 1) * fw / width) + ph)
    modes = (math.sqrt(2.0) * torch.cos(arg)).to(device)          # [S, n_modes]
    out = {}
    for name, tid in (("q", TENSOR_Q), ("k", TENSOR_K), ("v", TENSOR_V)):
        g = _gen(device, seed_of(stream, tid))
        zz = torch.randn((batch, heads, seq, head_dim), generator=g, device=device)
        w = torch.randn((heads, n_modes, head_dim), generator=g, device=device) / math.sqrt(n_modes)
        low = torch.matmul(modes, w)[None]          # [1, H, S, D]
        out[name] = (math.sqrt(1 - lam) * zz + math.sqrt(lam) * low).to(torch.bfloat16)
        del zz, low
    return out


def bf16_bits(t):
    """uint16 view of a bfloat16/float16 tensor as a numpy array (host copy)."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view("uint16")
