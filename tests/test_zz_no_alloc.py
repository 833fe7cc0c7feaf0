"""mxattn_decode_noalloc (the decode entry point that allocates nothing and
keeps its partial slots in the library's per-device scratch) against
mxattn_decode with a caller workspace: the same kernels, so the same bits.
Two calls in a row, the second smaller, so a stale first call's slots in the
shared scratch would show."""

import pytest
import torch

import bit_microscaled_flashattention_amd as mxa

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _workload(seed, b, hq, hkv, t, d, ctx):
    g = torch.Generator(device=DEV).manual_seed(seed)
    q = torch.randn((b, hq, d), generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn((b, hkv, t, d), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((b, hkv, t, d), generator=g, device=DEV).to(torch.bfloat16)
    return q, mxa.quantize(k, "hd"), mxa.quantize(v, "hd"), torch.tensor(ctx, dtype=torch.int32, device=DEV), k, v


def _hybrid(k, v, ctx, window, n_sel):
    b, hkv, t, d = k.shape
    idx = torch.full((b, hkv, n_sel), -1, dtype=torch.int32, device=DEV)
    n = torch.zeros((b, hkv), dtype=torch.int32, device=DEV)
    for bb in range(b):
        lim = int(ctx[bb]) - window
        sel = torch.arange(0, lim, max(lim // n_sel, 1), device=DEV)[:n_sel].to(torch.int32)
        idx[bb, :, :sel.numel()] = sel
        n[bb] = sel.numel()
    gidx = idx.clamp_min(0).long()[..., None].expand(-1, -1, -1, d)
    k_win = torch.stack([k[bb, :, int(ctx[bb]) - window:int(ctx[bb])] for bb in range(b)]).contiguous()
    v_win = torch.stack([v[bb, :, int(ctx[bb]) - window:int(ctx[bb])] for bb in range(b)]).contiguous()
    return {"idx": idx, "n_sel": n, "window": window, "k_sel": torch.gather(k, 2, gidx).contiguous(),
            "v_sel": torch.gather(v, 2, gidx).contiguous(), "k_win": k_win, "v_win": v_win}


def _both(q, kc, vc, ctx, split, hybrid=None):
    b, hq = q.shape[0], q.shape[1]
    d = kc.shape[3]
    ref_o, ref_l = mxa.decode(q, kc, vc, ctx, split_len=split, hybrid=hybrid, return_lse=True)
    out = torch.full((b, hq, d), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full((b, hq), float("nan"), dtype=torch.float32, device=DEV)
    mxa.decode_noalloc(q, kc, vc, ctx, out, split_len=split, hybrid=hybrid, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(ref_o, out) and torch.equal(ref_l, lse)


def test_noalloc_decode_matches_workspace_decode_twice():
    print("noalloc decode: batch 4, 32/8 heads, ctx 8192, split 1024", flush=True)
    q, kc, vc, ctx, _, _ = _workload(91, 4, 32, 8, 8192, 128, [8192, 5000, 4097, 64])
    _both(q, kc, vc, ctx, 1024)
    print("noalloc decode: smaller, batch 2, 8/2 heads, ctx 3000, split 256", flush=True)
    q, kc, vc, ctx, _, _ = _workload(92, 2, 8, 2, 3000, 128, [3000, 1234])
    _both(q, kc, vc, ctx, 256)


def test_noalloc_hybrid_decode_matches_twice():
    print("noalloc hybrid decode: batch 2, 32/8 heads, ctx 6000", flush=True)
    q, kc, vc, ctx, k, v = _workload(93, 2, 32, 8, 6000, 128, [6000, 4100])
    _both(q, kc, vc, ctx, 1024, _hybrid(k, v, ctx, 64, 200))
    print("noalloc hybrid decode: smaller, batch 1, 8/8 heads, ctx 700, d 64", flush=True)
    q, kc, vc, ctx, k, v = _workload(94, 1, 8, 8, 700, 64, [700])
    _both(q, kc, vc, ctx, 128, _hybrid(k, v, ctx, 16, 10))
