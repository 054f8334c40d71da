"""Tensor Cache second-level memory fed by evictions (oracle, fp64).

Test infrastructure (see the package docstring).

"Tensor Cache: Eviction-conditioned Associative Memory for Transformers"
(gist.science), section "Metodologia": the first level is a ring of the W
most recent key/value pairs with exact softmax attention; a pair the ring
overwrites is written into a fixed-size outer-product matrix A (per head),
A <- lambda A + eta (k outer v); a later query reads r = q A, which by the
linear-attention identity q (k outer v) = <q, k> v recovers every evicted
token's value weighted by its key's inner product with the query; the two
levels merge as y = y_local + sigmoid(g) r.

Readings taken here (the page's lambda, eta and g are learned per head; this
build has no weights, so they are fixed configuration scalars shared by all
heads):

* A is d x d per (sequence, layer, kv head), starts at zero, and is written
  only by tokens leaving the hot window, oldest first, one write per token;
  a query head h reads the matrix of its kv head h // (H_q / H_kv).
* The first level is this cache's hot window (FIFO, W entries after each
  append); y_local is exact softmax attention over it with logits
  <q, k>/sqrt(d).  m_t of the fusion is the read r_t.
* No promotion: A holds no individual tokens to bring back.
"""

import numpy as np

from . import attention as _att


def sigmoid(g: float) -> float:
    """Logistic function, evaluated without overflow for either sign."""
    if g >= 0:
        return 1.0 / (1.0 + np.exp(-g))
    e = np.exp(g)
    return e / (1.0 + e)


def write(A, k16, v16, lam: float, eta: float):
    """Sequential writes of n evicted tokens (k16, v16: [n, d], oldest first)
    into A [d, d]: A <- lam A + eta outer(k, v) per token.  Returns A."""
    A = np.array(A, dtype=np.float64)
    k = np.asarray(k16, dtype=np.float16).astype(np.float64)
    v = np.asarray(v16, dtype=np.float16).astype(np.float64)
    for t in range(k.shape[0]):
        A = lam * A + eta * np.outer(k[t], v[t])
    return A


def read(A, q16):
    """r = q A for query rows q16 [H, d] against one matrix A [d, d]."""
    return np.asarray(q16, dtype=np.float16).astype(np.float64) @ A


def decode_attention(q16, hot_k, hot_v, A, g: float):
    """y = softmax attention over the hot window + sigmoid(g) q A.

    q16 [H_q, d]; hot_k, hot_v [H_kv, n_hot, d] fp16; A [H_kv, d, d].
    Returns dict(out [H_q, d], local [H_q, d], read [H_q, d], logits_hot)."""
    q = np.asarray(q16, dtype=np.float16)
    hq, d = q.shape
    hkv = hot_k.shape[0]
    grp = hq // hkv
    n_hot = hot_k.shape[1]
    local = np.zeros((hq, d))
    rd = np.zeros((hq, d))
    lh = np.full((hq, n_hot), -np.inf)
    for kv in range(hkv):
        rows = slice(kv * grp, (kv + 1) * grp)
        if n_hot:
            lh[rows] = _att.hot_logits(q[rows].astype(np.float64), hot_k[kv])
            local[rows] = _att.softmax(lh[rows]) @ np.asarray(hot_v[kv], dtype=np.float16).astype(np.float64)
        rd[rows] = read(A[kv], q[rows])
    return dict(out=local + sigmoid(g) * rd, local=local, read=rd, logits_hot=lh)


class SeqLayerTC:
    """Hot window plus Tensor Cache matrix of one (sequence, layer)."""

    def __init__(self, n_kv_heads, d, window, lam, eta, g):
        self.hkv, self.d, self.W = n_kv_heads, d, window
        self.lam, self.eta, self.g = lam, eta, g
        self.hot_k = []  # FIFO of [H_kv, d] fp16
        self.hot_v = []
        self.A = np.zeros((n_kv_heads, d, d))
        self.n_written = 0

    def append(self, k16, v16):
        """Append n tokens ([n, H_kv, d] fp16); every token pushed out of the
        window is written into A, oldest first."""
        k16 = np.asarray(k16, dtype=np.float16)
        v16 = np.asarray(v16, dtype=np.float16)
        for t in range(k16.shape[0]):
            self.hot_k.append(k16[t].copy())
            self.hot_v.append(v16[t].copy())
        while len(self.hot_k) > self.W:
            k, v = self.hot_k.pop(0), self.hot_v.pop(0)
            for kv in range(self.hkv):
                self.A[kv] = write(self.A[kv], k[kv][None], v[kv][None], self.lam, self.eta)
            self.n_written += 1

    def hot_arrays(self):
        if not self.hot_k:
            z = np.zeros((self.hkv, 0, self.d), dtype=np.float16)
            return z, z
        return np.stack(self.hot_k, axis=1), np.stack(self.hot_v, axis=1)

    def attend(self, q16):
        hk, hv = self.hot_arrays()
        return decode_attention(q16, hk, hv, self.A, self.g)
