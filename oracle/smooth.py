"""Static per-channel Smooth-QK rescale.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "HiFA4: Training-Free 4-bit FlashAttention on Ascend HIF4 NPUs for LLM
Inference", Abstract: Smooth-QK is a calibration-static, per-channel,
equivalent rescaling of Q and K applied after RoPE that moves quantisation
difficulty from K to Q, with no per-tile reduction at inference time.  The
BitDecoding-FP4 page ("Outlier-Aware Key Quantization") describes the same
static smoothing: per-channel coefficients estimated in a calibration phase,
keys rescaled per channel.

Readings:
  * SmoothQuant form with strength 1/2: for KV head h and channel c,
        s = sqrt(kmax[h, c] / qmax[h, c])
    where kmax is max |K| over the calibration tokens and qmax is max |Q| over
    the calibration tokens and over the query heads that share KV head h.
    Q is multiplied by s and K by 1/s, so Q K^T is unchanged.
  * s is computed in float64 (one IEEE division, one IEEE square root), set to
    1 where either maximum is 0, clamped to [2^-8, 2^8]; the stored factors
    are float32(s) for Q and float32(1/s) for K.
  * The rescale itself is one IEEE float32 multiply (round to nearest even)
    of the float32 activation by the float32 factor.

Parity: pinned by tests/test_oracle_attention.py (with quantisation off the
smoothed attention equals the unsmoothed one; exactly for power-of-two s) and
tests/test_oracle_codec.py (hand-computed calibration case).
"""

import numpy as np

S_MIN, S_MAX = 2.0 ** -8, 2.0 ** 8


def calibrate(q_cal, k_cal):
    """Per-channel Smooth-QK factors from a calibration slice.

    q_cal: [Hq, T, D] values (any float dtype), k_cal: [Hkv, T, D].
    Returns (q_scale float32 [Hq, D], k_scale float32 [Hkv, D]).
    """
    q = np.abs(np.asarray(q_cal, dtype=np.float64))
    k = np.abs(np.asarray(k_cal, dtype=np.float64))
    hq, hkv = q.shape[0], k.shape[0]
    assert hq % hkv == 0
    g = hq // hkv
    qmax = q.max(axis=1).reshape(hkv, g, -1).max(axis=1)   # [Hkv, D]
    kmax = k.max(axis=1)                                    # [Hkv, D]
    with np.errstate(divide="ignore", invalid="ignore"):
        s = np.sqrt(kmax / qmax)
    s = np.where((qmax == 0) | (kmax == 0), 1.0, s)
    s = np.clip(s, S_MIN, S_MAX)
    k_scale = (1.0 / s).astype(np.float32)
    q_scale = np.repeat(s.astype(np.float32), g, axis=0)
    return q_scale, k_scale


def apply(x, chan_scale):
    """float32(x) * float32 factor per (head, channel); x: [..., H, S, D]."""
    x32 = np.asarray(x, dtype=np.float32)
    f = np.asarray(chan_scale, dtype=np.float32)[:, None, :]  # [H, 1, D]
    return (x32 * f).astype(np.float32)
