"""Vertical-line token selection for hybrid-precision decode.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "HyQuant: Hybrid-Precision Quantization for LLM Attention", method
paragraphs.  What this module implements from them: each key gets a score,
the attention probability it has received summed over columns of the
attention matrix; every few tokens the highest-scoring fraction rho of the
keys outside a fixed recent window is chosen to stay in full precision,
together with that window.

Readings
  * Column mass of key t gains, for every recent query r (at most 64, the
    queries decoded since the last selection) and every query head of the KV
    head's group, the softmax probability of t among all keys t' < ctx,
    computed from the MXFP4 query and MXFP4 keys.  Mass accumulates across
    calls with no decay.
  * Candidates are t in [0, ctx - W); k = ceil(n * rho_num / rho_den) with
    n = ctx - W, evaluated in integers so that rho = 5/100 gives exactly
    1632 of 32640.
  * Ties in mass go to the lower index; the result is sorted ascending.

Parity: pinned by tests/test_oracle_select.py (brute force over all subsets
on tiny inputs, the total-mass invariant: each recent query adds exactly one
unit of mass, and agreement with the decode softmax of oracle.attention).
"""

import numpy as np


def colmass_update(col_mass, q_hat, k_hat, ctx, softmax_scale=None):
    """col_mass [T] float64 (copied), q_hat [n_q, D], k_hat [T, D]."""
    cm = np.array(col_mass, dtype=np.float64, copy=True)
    q_hat = np.asarray(q_hat, dtype=np.float64)
    if q_hat.shape[0] == 0 or ctx == 0:
        return cm
    d = q_hat.shape[1]
    if softmax_scale is None:
        softmax_scale = 1.0 / np.sqrt(d)
    s = softmax_scale * (q_hat @ np.asarray(k_hat, dtype=np.float64)[:ctx].T)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    cm[:ctx] += p.sum(axis=0)
    return cm


def n_select(ctx, window, rho_num, rho_den):
    n = max(int(ctx) - int(window), 0)
    return (n * int(rho_num) + int(rho_den) - 1) // int(rho_den), n


def topk_vertical(col_mass, ctx, window, rho_num, rho_den):
    """Indices of the k heaviest non-window keys, ascending."""
    k, n = n_select(ctx, window, rho_num, rho_den)
    if k == 0:
        return np.zeros(0, dtype=np.int64)
    cm = np.asarray(col_mass, dtype=np.float64)[:n]
    order = np.lexsort((np.arange(n), -cm))      # mass descending, index ascending
    return np.sort(order[:k])


def select_vertical(col_mass, q_hat_recent, k_hat, ctx_len, window, rho_num, rho_den,
                    softmax_scale=None):
    """Multi-head selection.

    col_mass [B, Hkv, T]; q_hat_recent [B, Hq, R, D]; k_hat [B, Hkv, T, D].
    Returns (new col_mass [B, Hkv, T], {(b, hkv): idx ascending}).
    """
    bsz, hkv, _ = col_mass.shape
    hq, r = q_hat_recent.shape[1], q_hat_recent.shape[2]
    g = hq // hkv
    cm_out = np.array(col_mass, dtype=np.float64, copy=True)
    sel = {}
    for b in range(bsz):
        ctx = int(ctx_len[b])
        for h in range(hkv):
            qs = q_hat_recent[b, h * g:(h + 1) * g].reshape(g * r, -1)
            cm_out[b, h] = colmass_update(cm_out[b, h], qs, k_hat[b, h], ctx, softmax_scale)
            sel[(b, h)] = topk_vertical(cm_out[b, h], ctx, window, rho_num, rho_den)
    return cm_out, sel
