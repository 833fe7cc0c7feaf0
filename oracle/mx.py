"""MXFP4 codec: E2M1 elements sharing one E8M0 power-of-two scale per 32 values.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "BitDecoding-FP4: Algorithm-System Co-Design for Native FP4 KV Cache
Decoding", section "The KV Cache Bottleneck in Long-Context LLM Serving":
microscaling groups a tensor into fixed blocks (32 elements), every block
shares one E8M0 scaling factor, and the elements are FP4 E2M1.  The element
grid, the round-to-nearest-even rule and the shared-exponent rule of the
"direct" (OCP) baseline are those of the OCP Microscaling Formats v1.0
specification, which the MXAttention page names as its baseline ("OCP
MXFP4", Abstract).  The second scale rule is the Universal Optimal Scaling
bound of "MXAttention: Data-Free Optimal Scaling and Pre-Normalization
Quantization for MXFP4 Attention" (Abstract, AI Summary): a fixed boundary
Qmax = 7.25 on the block maximum measured in scale units.

Readings taken where the sources are silent:
  * E2M1 rounding is round-to-nearest, ties to the code whose mantissa bit is
    0; magnitudes above 6 saturate to 6; there is no Inf/NaN code.
  * A value that rounds to zero keeps its sign bit (code 0x8 for -0).
  * OCP rule: e = floor(log2 amax) - 2, so amax / 2^e lies in [4, 8).
  * UOS rule: e is the smallest integer with amax <= Qmax * 2^e, so amax / 2^e
    lies in (Qmax/2, Qmax].
  * e is clamped to [-127, 127]; an all-zero block gets e = -127 (byte 0);
    scale byte = e + 127, so byte 255 (NaN) is never produced.

Parity: pinned by tests/test_oracle_codec.py (closed forms, exhaustive bf16
enumeration against an independent threshold formulation, round trips, the
OCP/UOS boundary table in tests/golden/; bf16_bits_to_f64 against
hand-decoded bit patterns and the sign/exponent/mantissa formula; the
dual-residual split against its closed-form error bound).
"""

import numpy as np

# E2M1 magnitudes indexed by the low three code bits (OCP MX v1.0, FP4 E2M1:
# one sign bit, two exponent bits with bias 1, one mantissa bit).
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)

RULE_OCP = 0
RULE_UOS = 1
UOS_QMAX = 7.25          # MXAttention, Abstract: Qmax = 7.25
BLOCK = 32               # BitDecoding-FP4, "The KV Cache Bottleneck ...": blocks of 32
E_MIN, E_MAX = -127, 127  # E8M0 exponent range (byte 0..254)


def e2m1_decode(codes):
    """Value of each 4-bit code (bit 3 = sign, bits 0-2 = magnitude index)."""
    codes = np.asarray(codes, dtype=np.uint8)
    mag = E2M1_VALUES[codes & 7]
    return np.where(codes & 8, -mag, mag)


def e2m1_round_magnitude(mag):
    """Code (0..7) of the E2M1 magnitude nearest to ``mag`` (>= 0, float64).

    Nearest by absolute distance; when two grid points are equally near, the
    one with mantissa bit 0 (an even code) wins.  Values beyond 6 saturate.
    """
    # Saturation first: a magnitude beyond 6 codes as 6.  (Clipping also keeps
    # the distances below exact for huge inputs.)
    mag = np.minimum(np.asarray(mag, dtype=np.float64), E2M1_VALUES[-1])
    dist = np.abs(mag[..., None] - E2M1_VALUES)          # (..., 8)
    best = dist.min(axis=-1, keepdims=True)
    is_best = dist == best
    first = is_best.argmax(axis=-1)                       # lowest nearest code
    two = is_best.sum(axis=-1) == 2                       # a midpoint tie
    code = np.where(two & (first % 2 == 1), first + 1, first)
    return code.astype(np.uint8)


def e8m0_exponent(amax, rule=RULE_OCP, qmax=UOS_QMAX):
    """Shared block exponent e (scale 2^e) for block maxima ``amax`` (>= 0).

    OCP: e = floor(log2 amax) - 2 (E2M1's largest exponent is 2).
    UOS: the smallest integer e with amax <= qmax * 2^e.
    Both are evaluated exactly (frexp / ldexp / comparisons, no log2).
    """
    amax = np.asarray(amax, dtype=np.float64)
    mant, ex = np.frexp(amax)            # amax = mant * 2^ex, mant in [0.5, 1)
    floor_log2 = ex.astype(np.int64) - 1
    if rule == RULE_OCP:
        e = floor_log2 - 2
    elif rule == RULE_UOS:
        # Candidates around floor(log2(amax/qmax)); keep the smallest that fits.
        e = floor_log2 - 4
        for _ in range(6):
            fits = amax <= qmax * np.ldexp(1.0, e)
            e = np.where(fits, e, e + 1)
        # e now fits; step down while the next smaller exponent also fits.
        for _ in range(6):
            smaller_fits = amax <= qmax * np.ldexp(1.0, e - 1)
            e = np.where(smaller_fits, e - 1, e)
    else:
        raise ValueError("unknown scale rule")
    e = np.where(amax == 0, E_MIN, e)
    return np.clip(e, E_MIN, E_MAX).astype(np.int64)


def quantize_blocks(y, rule=RULE_OCP, qmax=UOS_QMAX):
    """MXFP4-quantise the last axis of ``y`` (length a multiple of 32).

    ``y`` holds the float32 values to encode (any float dtype; used exactly).
    Returns (codes uint8 same shape as y, scale bytes uint8 shape[:-1]+(n/32,)).
    """
    y = np.asarray(y, dtype=np.float64)
    n = y.shape[-1]
    assert n % BLOCK == 0, "block axis must be a multiple of 32"
    blocks = y.reshape(y.shape[:-1] + (n // BLOCK, BLOCK))
    amax = np.abs(blocks).max(axis=-1)
    e = e8m0_exponent(amax, rule, qmax)
    z = np.ldexp(np.abs(blocks), -e[..., None])      # exact power-of-two scaling
    mag_code = e2m1_round_magnitude(z)
    sign = np.signbit(blocks).astype(np.uint8) << 3
    codes = (mag_code | sign).reshape(y.shape)
    return codes, (e + 127).astype(np.uint8)


def dequantize_blocks(codes, scale_bytes):
    """Inverse of :func:`quantize_blocks` (exact in float64)."""
    codes = np.asarray(codes, dtype=np.uint8)
    n = codes.shape[-1]
    vals = e2m1_decode(codes).reshape(codes.shape[:-1] + (n // BLOCK, BLOCK))
    e = np.asarray(scale_bytes, dtype=np.int64) - 127
    return np.ldexp(vals, e[..., None]).reshape(codes.shape)


def quantize(x, axis, rule=RULE_OCP, qmax=UOS_QMAX):
    """Quantise ``x`` in 32-element blocks running along ``axis``.

    If the axis length is not a multiple of 32 the tail block is padded with
    +0, which neither raises the block maximum nor survives in the output.
    Returns (codes, scale bytes) with ``axis`` kept in place; the code array
    keeps the padded length, the scale array has ceil(n/32) entries on axis.
    """
    x = np.moveaxis(np.asarray(x, dtype=np.float64), axis, -1)
    n = x.shape[-1]
    pad = (-n) % BLOCK
    if pad:
        x = np.concatenate([x, np.zeros(x.shape[:-1] + (pad,))], axis=-1)
    codes, sb = quantize_blocks(x, rule, qmax)
    return np.moveaxis(codes, -1, axis), np.moveaxis(sb, -1, axis)


def dequantize(codes, scale_bytes, axis, n=None):
    """Inverse of :func:`quantize`; ``n`` trims the padded tail."""
    c = np.moveaxis(np.asarray(codes, dtype=np.uint8), axis, -1)
    s = np.moveaxis(np.asarray(scale_bytes, dtype=np.uint8), axis, -1)
    v = dequantize_blocks(c, s)
    if n is not None:
        v = v[..., :n]
    return np.moveaxis(v, -1, axis)


def quantize_dual(x, axis, rule=RULE_OCP, qmax=UOS_QMAX):
    """Dual-residual MXFP4: ``x`` ~ dequant(q1) + dequant(q2).

    Source: BitDecoding-FP4, section "Dual-Residual Query Quantization": the
    query is split into two FP4 tensors so that more of it survives than in
    one, at no extra cache storage (only the query is split).  Reading (the
    page does not print the split): q1 = MXFP4(x) and q2 = MXFP4(x -
    dequant(q1)), both with the same block axis and scale rule.  The residual
    is exact here (float64) and also in float32, because dequant(q1) is 0 or
    within a factor of two of x (Sterbenz), so an fp32 implementation forms
    the same residual bit for bit.
    Returns (codes1, scales1, codes2, scales2) as :func:`quantize`.
    """
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[axis]
    c1, s1 = quantize(x, axis, rule, qmax)
    r = x - dequantize(c1, s1, axis, n)
    c2, s2 = quantize(r, axis, rule, qmax)
    return c1, s1, c2, s2


def pack_nibbles(codes, axis=-1):
    """Two codes per byte along ``axis``: element 2j low nibble, 2j+1 high."""
    c = np.moveaxis(np.asarray(codes, dtype=np.uint8), axis, -1)
    assert c.shape[-1] % 2 == 0
    packed = (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)
    return np.moveaxis(packed.astype(np.uint8), -1, axis)


def unpack_nibbles(packed, axis=-1):
    p = np.moveaxis(np.asarray(packed, dtype=np.uint8), axis, -1)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return np.moveaxis(out, -1, axis)


def bf16_bits_to_f64(bits):
    """Exact value of bfloat16 bit patterns (uint16) as float64: the pattern
    is the upper half of a float32 whose lower 16 bits are zero."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)
