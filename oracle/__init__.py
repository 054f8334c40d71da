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
* "Compresion del cache KV de los LLM a 3 bits: TurboQuant" (sudonull.com,
  Spanish) -- section "Aplicaciones mas alla de los LLMs" (the codec applied
  to vector search).
* "Tensor Cache: Eviction-conditioned Associative Memory for Transformers"
  (gist.science) -- section "Metodologia" (a second-level outer-product
  memory written by the tokens the window evicts, read as q A, merged through
  a gate).

Where the pages leave a step open the oracle takes one explicit reading and
states it in the docstring of the function that takes it.

Parity status per function (what pins it, see tests/test_oracle_*.py):

* params.splitmix64 / uniforms / normals: published SplitMix64 test outputs,
  Box-Muller closed form on hand-picked uniforms, moment checks.
* params.rotation: orthogonality, norm and inner-product preservation,
  QR uniqueness against an independent Gram-Schmidt.
* params.hadamard_rotation: orthogonal, equal to the closed-form Walsh matrix
  times the published generator's signs.
* attention.decode_attention(gate=theta) (the hot-first gate): theta = +inf
  is the plain step, theta = -inf leaves hot-only attention equal to torch's
  SDPA over the window; planted hot keys gate exactly the kv groups whose
  every head reaches theta (a group with one head below stays open and equals
  the ungated step); lowering theta never reopens a group.
* attention.multi_query_attention: one query is the decode step; without cold
  tokens it equals torch's SDPA with the causal chunk mask; earlier queries
  never see later chunk tokens.
* codec.*: hand-worked codes with the identity rotation, brute-force nearest
  codeword, per-pair error bounds, closed-form byte counts, MSE falling with
  bit width, QJL unbiasedness and closed-form variance over 10k sketches.
* codec.dequantize / codec.qjl_backprojection and attention.cold_logits (the
  QJL term as decode computes it): over 10k sketches the compressed logit and
  <q, x_hat> are unbiased estimates of the exact logit <q, x>/sqrt(d), with
  the sign estimator's closed-form spread; the mean of x_hat is x with the
  closed-form total variance.
* codec.boundary_band: equal, field by field, to a brute-force geometric
  reading (distance to every decision half-line and radius threshold circle,
  distance to fp16 rounding midpoints, |z_j| against tol |S_j|) at two band
  widths, plus planted ties on decision rays and non-ties on grid angles.
* attention.*: identity between the code-domain logit and the brute-force
  logit on dequantised keys; hot-only attention against torch's SDPA on CPU;
  split-K merge equals one pass; permutation invariance.
* mips.*: the score equals the inner product with the dequantised vector,
  the selection equals a brute-force sort (ties, tombstones, padding), a fine
  code converges to exact search, and recall@10 rises with the bit width.
* tensor_cache.*: the read equals linear attention over exactly the evicted
  tokens (the page's identity q (k outer v) = <q, k> v), blocked writes equal
  sequential ones, only tokens leaving the window reach the matrix, and a
  closed gate leaves window-only softmax attention (torch SDPA on CPU).
* paging.*: brute-force invariants (every token live exactly once, window
  bound, FIFO order) and planted heavy hitters promoting on exactly the
  sticky-th qualifying step.
* The pages' model-quality numbers (perplexity, LongBench, RULER, NIAH, ANN
  recall) need models and datasets that are absent: parity unpinned, and no
  function here claims them.
"""

from . import params, codec, attention, paging, tensor_cache, mips  # noqa: F401
