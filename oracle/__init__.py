"""CPU oracle for the WUSH online path.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product (``mxfp4_activation_amd``)
never imports it.  The two share no code.  They share only the seeded
generators in ``synthetic``, which contain none of the method's arithmetic.

What it follows (source pages: "WUSH: Near-Optimal Adaptive Transforms for LLM
Quantization", arXiv 2512.00956):

* ``transform``  builds the offline per-block transforms.  The blockwise
  second moments come from the papernotes.org summary, "整体框架" / "关键设计",
  and the paper-graph deep dive, sections 3.2 and 3.4.2.  The Cholesky
  factors and the SVD of W'^T X' are Eq. 7.  T_wush = H S^-1/2 U^T W'^T and
  T_xvsh = H S^-1/2 V^T X'^T are Eq. 8 in section 3.4.4.
* ``codecs``     holds the 4-bit element grids and their scale encodings:
  E2M1 with an E8M0 scale (MXFP4), E2M1 with an E4M3 scale (NVFP4), and
  symmetric INT4 with an fp16 scale.  The pages name these formats but
  do not spell out their encodings.  The encodings here are the standard
  OCP MX / OCP FP8 / IEEE binary16 definitions.
* ``gemm``       is the FP4 matrix product that consumes the quantized
  activations and the pre-quantized weights (deep dive, section 3.4.6,
  Eq. 10): decode both MXFP4 operands, multiply in float64.
* ``gptq``       is GPTQ-WUSH, Algorithm 1 (deep dive, section 3.4.6): the
  weight side calibrated block by block in reverse order, with the
  transform rebuilt from the residual target before each block's GPTQ.
* ``loss``       is the layerwise loss of Eq. 5 (deep dive, section 3.4.1):
  quantize both operands through their block transforms, multiply, and
  take the mean squared error against the unquantized product.
* ``quant``      is the online path.  For every token and block it computes
  y = T_wush(c) x.  Then it applies RTN AbsMax quantization of y in groups
  of G, the transform block (deep dive, sections 3.4.1 and 3.4.7; Eq. 10).

Readings where the pages are silent are stated where they are used.  The
list:
  - The SVD sign freedom is fixed by making each right singular vector's
    largest-magnitude entry positive.
  - Damping is lambda * mean(diag) * I on both moments, with lambda = 1e-6.
  - The Hadamard matrix is in Sylvester order, scaled by G^-1/2.
  - y is the exact sum rounded once to fp32.
  - The MXFP4 shared exponent is floor(log2 amax) - 2, clamped to [-127, 127].
  - Element rounding is to nearest, ties to even, saturating.
  - NVFP4 and INT4 divide by their scale by multiplying with the correctly
    rounded fp32 reciprocal.
  - Element 2j goes in the low nibble of byte j.

Parity unpinned: the transform's bytes cannot be compared against the
authors' implementation, because their code is not available.  Their sign,
ordering and damping choices may differ from the readings above.
"""
