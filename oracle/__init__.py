"""CPU oracle for the smoothed, outlier-split, dual-branch W4A4 linear layer.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
NumPy implementation of what the layer computes.  Only the test suite, the
smoke check and the benchmark's CPU-baseline leg may import it; the product
path (``mixed_gemm_amd``) never does, and this package imports nothing from it.

Source: "W4A4 Quantization for Inference on Wan2.2-I2V-A14B" (arXiv
2606.29337), in particular

* Eq. (1)  the SmoothQuant fold  Y = (X / s)(s * W), applied along input channels;
* Eq. (2)  s_j = act_scale_j^alpha / weight_scale_j^(1 - alpha);
* Eq. (4)  score_j = max_t |x_tj| and the top-k outlier column set O;
* Eq. (5)  Y = X_J W^(q)_J + X_O W^(hp)_O (Eq. (3) with a static O): a W4A4
  bulk branch over the remaining columns J plus a high-precision branch;
* the calibration, integration and block-packing paragraphs that follow those
  equations (per-input-channel activation maxima and weight column ranges, the
  fold before packing, O kept as sparse index lists, activations divided by s
  just before the 4-bit quantize, 1x32 / 32x32 block scales).

MXFP4 is taken as E2M1 elements with one E8M0 power-of-two scale per block of
32, following the OCP Microscaling rules (shared exponent = floor(log2 amax)
minus the element format's emax of 2; elements rounded to nearest, ties to
the even code, saturating at +-6).

Every function in ``oracle.layer`` and ``oracle.mxfp4`` is pinned by a
``-m "not gpu"`` test against something other than itself (brute force,
closed forms, exact rational arithmetic, special cases).  ``gelu_tanh`` is
pinned against the closed form evaluated with ``math.tanh``.
"""
from . import mxfp4, layer  # noqa: F401
