"""Plain CPU oracle for 4-bit block-scaled (MXFP4) FlashAttention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link this package: only the tests, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code, table or helper with the HIP
library; the two meet only through the seeded input generators in ``synth``.

Everything here is numpy.  Integer work (codes, scale bytes, indices) is exact;
attention arithmetic runs in float64.  The float32 steps are the Smooth-QK
channel multiply, which the method defines on float32 activations, and the
Hadamard rotation that feeds the quantiser.

Modules
  mx         -- E2M1 element / E8M0 scale codec (OCP rule and the UOS bound)
  smooth     -- static per-channel Smooth-QK calibration and rescale
  attention  -- tiled online-softmax prefill with pre-normalisation P
                quantisation, and the (hybrid) decode softmax
  select     -- accumulated column mass and top-rho vertical-line selection
  rotate     -- Hadamard rotation of query/key rows before quantisation

Parity status per function is stated in each module's header.
"""

from . import mx, smooth, attention, select, rotate  # noqa: F401
