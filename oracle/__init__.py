"""CPU oracle for the rotated low-bit linear layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import or call anything in
this package.  The product path (the HIP library and its Python binding) never
imports it, and this package imports nothing from the product path.

Everything here is a plain, slow, obviously-correct NumPy implementation of
what the layer computes, written from the pages:

  * OrbitQuant PR #25 ("Default changes", "Runtime work"): randomly permuted
    block-Hadamard (RPBH) rotation, independent extra rounds, absmax INT8
    activations, dense block-Hadamard matrix form of the rotation;
  * CentriQ (arXiv 2610.06260), Sec. 3 "Preliminaries" (Eq. 1 activation
    quantizer, Hadamard facts, Lemma 1), Sec. 4.2 "Activation path" (Eq. 4
    exact centering and rank-1 restore, Eq. 5 forward pass, Eq. 6 offset
    invariance), App. B.2 (Eq. 9 epilogue), App. C.5 (Eq. 10 row-sum split);
  * Pith review of WUSH (arXiv 2512.00956), "Core claim": per-block transform
    pair with T_x = T_w^{-T}, RTN absmax MXFP4 block quantizers with G = 32;
  * FLUX.1-schnell-OrbitQuant-W4A4 model card, "Quantization" table: rotation
    rpbh, activation normalization epsilon 1e-10, codebook lloyd_max;
  * OrbitQuant PR #25 ("Default changes") and CentriQ Sec. 2 ("Related work"):
    Lloyd-Max activation codes from the post-rotation marginal.

Floating point: values are computed in float64 (the mathematics) and, where
the integer codes depend on float32 rounding, in one fixed float32 evaluation
order (the "canonical float32" result) that the codes are defined by.

Modules:
  hadamard  Sylvester matrices, dense and staged fast Walsh-Hadamard transforms
  rotation  RPBH rounds and per-32 dense transforms
  quant     mean, centering, absmax integer codes, INT4 packing, MXFP4 codec
  gemm      grouped integer products, fp32-scale epilogue, MXFP4 product
  linear    offline weight preparation and the whole forward pass
  lloyd_max Lloyd-Max codebook of the sphere marginal, nearest-level codes,
            the float16 dequantizing product
  asym      asymmetric grouped INT4 weights (CentriQ Eq. 2, App. B.2): RTN
            min-max scale and shift, stored offset codes, the corrected product
  kron      the factorised Paley x Sylvester rotation with zero padding
            (CentriQ Sec. 4.2 "Rotation", App. B.1)
"""
from . import hadamard, rotation, quant, gemm, linear, lloyd_max, asym, kron  # noqa: F401
