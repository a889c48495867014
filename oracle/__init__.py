"""Plain CPU oracle for TurboQuant KV-cache quantization and decode attention.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and the cpu_baseline
leg of bench.py may import or run anything in this package. The library
(decode_attention_tq_amd) never imports it and shares no code with it.

Everything is float64 NumPy, written from the method as the pages describe it:

* ai-accelerate.xyz TurboQuant article, section "TurboQuantの仕組み", step 1
  (PolarQuant): multiply each KV vector by a random orthogonal matrix so every
  coordinate becomes close to Gaussian, then quantize each coordinate on its own
  with the optimal (Lloyd-Max) scalar quantizer; no per-block full-precision
  scale or centroid is kept.
* same article and section, step 2 (QJL): one sign bit of a Johnson-Lindenstrauss
  projection of the remaining error makes the inner-product estimate unbiased;
  the qxai.app article on Tether QVAC's TurboQuant describes the same three parts
  (random rotation, scalar quantization, 1-bit QJL on the residual).

Where the pages leave a step open (random generator, code order, bit layout,
norm storage, attention scale) the reading taken is stated in the module that
implements the step.

Modules:
  rng        SplitMix64 counter generator, uniforms, Box-Muller normals
  rotation   seeded Gaussian matrix and Haar rotation (QR with sign fix)
  codebook   Gaussian Lloyd-Max codebook, fp16-rounded canonical form, MSE
  quantize   norm, rotate, threshold rule, bit packing (key and value layouts), QJL
  attention  dequantize, textbook decode attention, rotated-domain decode, split merge
"""
from . import rng, rotation, codebook, quantize, attention  # noqa: F401
