"""Launch-bound calls replayed from a captured HIP graph.

The library's entry points launch on the caller's stream and allocate
nothing when their outputs and workspace are passed in, so a whole step can
be captured once and replayed.  Each replay runs on new input values written
in place, with eager work and a synchronisation between replays, and must
equal the eager call on the same inputs bit for bit.
"""
import pytest
import torch

import bit_microscaled_flashattention_amd as mxa
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _capture(fn):
    """Warm fn up on a side stream, then capture one call of it."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_graph_replay_quantise_and_prefill():
    """The small prefill step (quantise Q, K, V in one launch + attention)."""
    d = synth.tiny(device=DEV)
    q, k, v = d["q"].clone(), d["k"].clone(), d["v"].clone()
    out = torch.empty((1, 1, 128, 64), dtype=torch.float32, device=DEV)
    qh, kh = mxa.empty_mx((1, 1, 128, 64), "hd"), mxa.empty_mx((1, 1, 128, 64), "hd")
    vh = mxa.empty_mx((1, 1, 128, 64), "key")
    jobs = [dict(x=q, out=qh), dict(x=k, out=kh), dict(x=v, layout="key", out=vh)]

    def step():
        mxa.quantize_batch(jobs)
        mxa.prefill(qh, kh, vh, causal=False, out=out)

    print("graph: tiny quantise + prefill", flush=True)
    g = _capture(step)
    gen = torch.Generator(device=DEV).manual_seed(71)
    for rep in range(4):
        for t in (q, k, v):
            t.copy_(torch.randn(t.shape, generator=gen, device=DEV).to(t.dtype))
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        step()
        torch.cuda.synchronize()
        assert torch.equal(got, out), f"replay {rep} differs from the eager step"


def test_graph_replay_decode_with_workspace():
    """A split decode call with its workspace passed in (scan + merge)."""
    gen = torch.Generator(device=DEV).manual_seed(73)
    b, hq, hkv, tcap, dim, split = 2, 8, 2, 1500, 128, 512
    kc = mxa.quantize(torch.randn((b, hkv, tcap, dim), generator=gen, device=DEV).to(torch.bfloat16), "hd")
    vc = mxa.quantize(torch.randn((b, hkv, tcap, dim), generator=gen, device=DEV).to(torch.bfloat16), "hd")
    q = torch.randn((b, hq, dim), generator=gen, device=DEV).to(torch.bfloat16)
    ctx = torch.tensor([1500, 777], dtype=torch.int32, device=DEV)
    ws = torch.empty(mxa.decode_workspace_bytes(b, hq, hkv, dim, tcap, split), dtype=torch.uint8, device=DEV)
    out = torch.empty((b, hq, dim), dtype=torch.float32, device=DEV)

    def call():
        mxa.decode(q, kc, vc, ctx, split_len=split, workspace=ws, out=out)

    print("graph: decode with workspace", flush=True)
    g = _capture(call)
    for rep in range(4):
        q.copy_(torch.randn(q.shape, generator=gen, device=DEV).to(q.dtype))
        ctx.copy_(torch.tensor([1500 - 100 * rep, 777 + 50 * rep], dtype=torch.int32, device=DEV))
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        call()
        torch.cuda.synchronize()
        assert torch.equal(got, out), f"replay {rep} differs from the eager call"
