"""CPU oracle for TurboQuant-style two-stage KV compression and attention over the codes.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and its Python
binding) may import, call or link anything in this package.  Only the test suite, the
smoke check and the CPU-baseline leg of the benchmark use it.

The oracle is written from the method's description on five web pages:

* "KV cache está consumiendo tu VRAM ... TurboQuant" (7minutos.es) -- stage 1 (random
  rotation, Beta law of a rotated coordinate, Lloyd-Max codebook, index storage),
  stage 2 (residual, QJL sign sketch, residual norm, unbiased QJL dequantisation);
* "TurboESM: Ultra-Efficient 3-Bit KV Cache Quantization for Protein Language Models"
  (gist.science, Spanish and Korean summaries) -- RoPE before the rotation, per-head
  rotations, fused decode attention over the compressed cache;
* "TurboQuant: compresión 6x de LLM KV-cache" (sudonull.com) and the hada.io TurboQuant
  news page -- norm/direction split, query kept in high precision, vector search.

It is plain and slow on purpose: fp64 arithmetic for everything that is an estimate,
IEEE fp32 per-operation rounding (NumPy never fuses multiply-add) for the steps whose
fp32 results decide stored integers, and exact arithmetic (``math.fsum``,
``fractions.Fraction``) wherever a stored bit is defined by an exact real quantity.

Modules
-------
rng       SplitMix64 + Box-Muller, the counter-based generator both sides implement.
codec     Haar rotation, Gaussian sketch, Lloyd-Max codebook for the rotated-coordinate law.
quantize  encode: norm, index, residual, QJL signs, bit packing.
estimate  score estimator, attention over dequantised K/V, inner-product top-k search.

Parity unpinned: nothing.  Every public function is pinned by a test in
``tests/test_oracle_*.py`` against a closed form, a textbook table, a worked example
from the pages, an invariant or brute force.
"""

from . import rng, codec, quantize, estimate  # noqa: F401
