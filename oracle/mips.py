"""Maximum inner-product search over compressed vectors (oracle, fp64).

Test infrastructure (see the package docstring).

"Compresion del cache KV de los LLM a 3 bits: TurboQuant" (sudonull.com,
Spanish), section "Aplicaciones mas alla de los LLMs", and "TurboQuant:
kompresja KV-cache w LLM 6 razy" (sudonull.com, Polish), section
"Zastosowanie poza LLM": the same codec serves vector search -- database
vectors are stored as codes and a query's inner products are estimated
from them.  Readings taken here:

* The score of stored vector j for query q is the code-domain estimate the
  decode path uses for a cold key, <q, x_hat_j> = <q', y_hat_j> +
  sqrt(pi/2)/m rho_j <S_m q', sigma_j> with q' = Pi q (no 1/sqrt(d) scale).
* The result is the k highest scores per query, in descending order, ties
  broken by the lower slot; tombstoned slots are not candidates.
"""

import numpy as np

from . import attention as _att
from .codec import Format


def scores(q16, codes, pi, s_full, fmt: Format) -> np.ndarray:
    """Estimated inner products [n_q, N] of queries q16 [n_q, d] against the
    N coded vectors."""
    q = np.asarray(q16, dtype=np.float16).astype(np.float64)
    return _att.cold_logits(q, codes, pi, s_full, fmt) * np.sqrt(q.shape[1])


def topk(sc: np.ndarray, k: int, live=None):
    """(indices [n_q, k], scores [n_q, k]): the k best of each row, score
    descending then slot ascending; -1 / -inf pad rows with fewer than k
    candidates."""
    sc = np.asarray(sc, dtype=np.float64)
    n_q, n = sc.shape
    if live is not None:
        sc = np.where(np.asarray(live, dtype=bool)[None, :], sc, -np.inf)
    idx = np.full((n_q, k), -1, dtype=np.int64)
    val = np.full((n_q, k), -np.inf)
    slots = np.arange(n)
    for r in range(n_q):
        ok = np.isfinite(sc[r])
        order = np.lexsort((slots[ok], -sc[r][ok]))  # primary: score descending; then slot
        take = min(k, order.size)
        idx[r, :take] = slots[ok][order[:take]]
        val[r, :take] = sc[r][ok][order[:take]]
    return idx, val


def exact_topk(q16, x16, k: int):
    """The uncompressed baseline: top-k of <q, x> over fp16 vectors x16 [N, d]."""
    q = np.asarray(q16, dtype=np.float16).astype(np.float64)
    x = np.asarray(x16, dtype=np.float16).astype(np.float64)
    return topk(q @ x.T, k)


def recall_at(found: np.ndarray, truth: np.ndarray) -> float:
    """Mean over queries of |found_r intersect truth_r| / |truth_r|."""
    hits = [len(set(f.tolist()) & set(t.tolist())) / max(1, len(t)) for f, t in zip(found, truth)]
    return float(np.mean(hits))
