"""CPU oracle for the RotorQuant / TurboQuant KV-vector codec.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, float64 numpy
statement of what the codec computes.  Only the test-suite, the smoke check
in ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import it.  The product path (the HIP library and its Python binding)
never imports, links or calls anything here, and nothing here imports the
product path: the two share no code, no tables and no constants.

Modules
-------
prng       SplitMix64 streams, uniforms and Box-Muller normals (the
           parameter draws; each side implements the published generator).
clifford   Cl(3,0) geometric algebra: full 8x8 product, reverse, rotors,
           the sandwich (R v) R~ as two explicit products.
lloyd_max  Lloyd-Max scalar quantizer for the coordinate density of a
           uniformly random unit vector (Beta-type density), plus the
           Gaussian N(0, 1/d_eff) variant.
params     Parameter tables from (d, bits, seed, mode): rotors, codebook,
           Pi (Gram-Schmidt QR), S.
codec      Quantize / dequantize / q.k estimate for RotorQuant and
           TurboQuant, MSE-only and with the QJL residual stage; bit packing.
theory     Closed forms the pages state (bounds, counts, constants).

Sources (the pages):
  RotorQuant README "TurboQuant + RotorQuant" (git mirror of
  scrya-com/rotorquant): sections "How TurboQuant Works", "How RotorQuant
  Works", "FMA Count", "Codebook Calibration Fix", "The Fused CUDA Kernel",
  "Non-Commutative Algebra Bug Fix", "MSE Quality".
  Blog "TurboQuant 论文解读": sections on normalisation, random rotation
  (Lemma 1), Beta distribution, Theorem 1, QJL (Lemma 4 / Theorem 2),
  Theorem 3, and the numpy demo.
  hyper.ai summary of arXiv 2504.19874, section "方法" (Algorithms 1 and 2).
"""
