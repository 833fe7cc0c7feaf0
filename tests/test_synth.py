"""The synthetic workloads have the structure their descriptions promise
(checked on the CPU; the hybrid-decode bias through the oracle)."""

import numpy as np
import torch

import synth
from oracle import mx, select


def test_outlier_channels_of_gqa_prefill():
    d = synth.gqa_prefill(device="cpu", seq=512)
    k = d["k"].float()[0]                                   # [Hkv, S, D]
    std = k.std(dim=1)                                      # [Hkv, D]
    for h, chans in enumerate(d["outlier_channels"]):
        assert (std[h, chans] > 9).all()
        mask = torch.ones(128, dtype=torch.bool)
        mask[chans] = False
        assert (std[h, mask] < 1.3).all()
    assert d["q_cal"].shape == (32, 256, 128) and d["k_cal"].shape == (8, 256, 128)


def test_hybrid_decode_vertical_line_mass():
    """Top 5% of the non-window keys hold 50-70% of the recent queries' mass
    (mean over KV heads), computed by the oracle on the MXFP4 operands."""
    d = synth.hybrid_decode(device="cpu", batch=1)
    fracs = []
    for h in range(8):
        kc, ks = mx.quantize(d["k"][0, h].double().numpy(), axis=1)
        kd = mx.dequantize(kc, ks, axis=1)
        q = d["q_recent"][0, 4 * h:4 * h + 4].double().numpy().reshape(-1, 128)
        qc, qs = mx.quantize(q, axis=1)
        cm = select.colmass_update(np.zeros(32768), mx.dequantize(qc, qs, axis=1), kd, 32768)
        top = np.sort(cm[:32640])[::-1]
        fracs.append(top[:1632].sum() / cm.sum())
    assert 0.5 <= np.mean(fracs) <= 0.7, fracs


def test_diffusion_low_rank_structure():
    d = synth.diffusion(device="cpu", heads=2, frames=2, height=16, width=16)
    q = d["q"].float()[0, 0]                                 # [S, D]
    # The shared low-frequency part makes neighbouring tokens correlated;
    # independent noise alone would not.
    near = torch.corrcoef(torch.stack([q[:-1].flatten(), q[1:].flatten()]))[0, 1]
    perm = torch.randperm(q.shape[0], generator=torch.Generator().manual_seed(0))
    far = torch.corrcoef(torch.stack([q.flatten(), q[perm].flatten()]))[0, 1]
    assert near > 0.15 and abs(far) < near / 2
    assert abs(q.std().item() - 1.0) < 0.1
