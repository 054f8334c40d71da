"""CPU oracle for compressed-KV decode (test infrastructure, not product code).

Plain, slow, fp64 numpy implementation of what the compressed-KV decode path
computes: the seeded random rotation and sign sketch, PolarQuant pair codes,
the QJL 1-bit residual sketch, decode attention read straight from the codes,
and Monarch-style hot/cold paging with sticky promotion.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It imports nothing from the HIP library
or its Python binding, and the library imports nothing from here.

Sources (page titles as printed on the web pages that describe the method):

* "TurboQuant: kompresja KV-cache w LLM 6 razy bez utraty dokladnosci"
  (sudonull.com, Polish) -- section "Zasada dzialania PolarQuant" (rotation
  then polar coordinates then quantisation) and section "Kompensacja bledow
  przez QJL" (1-bit JL sketch of the residual).
* "TurboQuant: optimizacion de memoria para KV caches en inferencia de LLMs"
  (kerneldigest.dev) -- sections "Arquitectura del Sistema" and the seven-step
  quantisation flow (polar map, polar quantisation, QJL correction, compressed
  store, attention logits from the compressed cache).
* "Monarch v3: Paginacion KV Inspirada en NES" (openclawradar.com) -- sections
  "Como funciona" (hot/cold regions, sliding-window eviction,
  attention-weighted promotion with a sticky mechanism) and "Bucle de
  Decodificacion Simplificado" (attend, promote, evict oldest to cold).

Where the pages leave a step open the oracle takes one explicit reading and
states it in the docstring of the function that takes it.

Parity status per function (what pins it, see tests/test_oracle_*.py):

* params.splitmix64 / uniforms / normals: published SplitMix64 test outputs,
  Box-Muller closed form on hand-picked uniforms, moment checks.
* params.rotation: orthogonality, norm and inner-product preservation,
  QR uniqueness against an independent Gram-Schmidt.
* codec.*: hand-worked codes with the identity rotation, brute-force nearest
  codeword, per-pair error bounds, closed-form byte counts, MSE falling with
  bit width, QJL unbiasedness and closed-form variance over 10k sketches.
* attention.*: identity between the code-domain logit and the brute-force
  logit on dequantised keys; hot-only attention against torch's SDPA on CPU;
  split-K merge equals one pass; permutation invariance.
* paging.*: brute-force invariants (every token live exactly once, window
  bound, FIFO order) and planted heavy hitters promoting on exactly the
  sticky-th qualifying step.
* The pages' model-quality numbers (perplexity, LongBench, RULER, NIAH, ANN
  recall) need models and datasets that are absent: parity unpinned, and no
  function here claims them.
"""

from . import params, codec, attention, paging  # noqa: F401
