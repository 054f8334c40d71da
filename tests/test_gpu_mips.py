"""Compressed-vector maximum inner-product search on the GPU against the
oracle ("Compresion del cache KV de los LLM a 3 bits: TurboQuant",
sudonull.com, section "Aplicaciones mas alla de los LLMs"): synthetic
Gaussian database vectors stored through the cache's own quantiser, top-k
of the code-domain inner products per query."""

import numpy as np
import pytest

from compressed_kv_decode_amd import tqkv
from oracle import codec, mips, params

from gpu_helpers import check_codes, dev, fmt_of

pytestmark = pytest.mark.gpu


def _store(n, d, fmt, seed, **over):
    """A 1-kv-head cache whose cold slots 0 .. n-1 hold n seeded vectors."""
    import torch
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((n, 1, d)) * rng.choice([0.5, 1.0, 3.0], size=(n, 1, 1))).astype(np.float16)
    c = tqkv.Cache(n_seq_max=1, n_layers=1, n_q_heads=1, n_kv_heads=1, head_dim=d, hot_window=64, max_context=n,
                   formats=[fmt], seed=seed, **over)
    zeros = np.zeros_like(x)
    c.append(0, [0], [n], dev(x), dev(zeros))
    c.evict(0, [0], 0)
    torch.cuda.synchronize()
    assert c.stats(0, 0)["cold_len"] == n
    return c, x[:, 0]


def _check(c, x, fmt, d, seed, n_q, k):
    import torch
    rng = np.random.default_rng(seed + 1)
    q = rng.standard_normal((n_q, d)).astype(np.float16)
    idx, sc = c.mips_search(0, 0, 0, dev(q), k)
    torch.cuda.synchronize()
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    pi, s = params.rotation(d, seed), params.sketch(64, d, seed)
    fm = fmt_of(fmt)
    codes, _, _ = check_codes(c.export_codes(0, 0, 0, 0, 0, x.shape[0]), x, pi, s, fm, d, "store")
    want_s = mips.scores(q, codes, pi, s, fm)
    wi, wv = mips.topk(want_s, k)
    # the logit bar 1e-3 max(|l|, 1) with l = score / sqrt(d), in score units
    tol = 1e-3 * np.maximum(np.abs(wv[:, -1:]), np.sqrt(d))
    for r in range(n_q):
        got = idx[r]
        assert np.all(got >= 0)
        # every returned slot's oracle score reaches the k-th best (within the tolerance)
        assert np.all(want_s[r, got] >= wv[r, -1] - tol[r]), f"query {r}: a returned slot is below the k-th best"
        # the scores agree with the oracle's for the same slots and come sorted
        assert np.all(np.abs(sc[r] - want_s[r, got]) <= tol[r]), f"query {r}: scores"
        assert np.all(np.diff(sc[r]) <= 0)
        # the sets differ only where scores tie within the tolerance
        miss = set(wi[r].tolist()) - set(got.tolist())
        for j in miss:
            assert want_s[r, j] <= wv[r, -1] + tol[r], f"query {r}: slot {j} missing"
    return idx, wi


@pytest.mark.parametrize("fmt,d,n", [((2, 3, 32), 128, 20000), ((3, 4, 64), 128, 7777), ((2, 2, 64), 64, 3001)])
def test_mips_topk_against_oracle(fmt, d, n):
    c, x = _store(n, d, fmt, seed=9)
    for n_q, k in ((8, 10), (13, 32), (1, 1)):
        _check(c, x, fmt, d, 9, n_q, k)


def test_mips_skips_tombstoned_slots_and_pads():
    """A stored vector that attention promotes back to hot leaves its slot
    tombstoned: the search skips it.  A store with fewer than k vectors pads
    with -1 / -inf."""
    import torch
    d = 64
    c, x = _store(20, d, (2, 3, 32), seed=4, promote_threshold=1.0 / 64, sticky=1)
    j = 7
    q = (x[j].astype(np.float32) * 3.0).astype(np.float16)[None]  # attention on slot 7
    c.attend(0, [0], dev(q[None]))
    c.promote(0, [0])
    torch.cuda.synchronize()
    live, _ = c.export_paging(0, 0, 20)
    assert not live[j] and live.sum() < 20
    idx, sc = c.mips_search(0, 0, 0, dev(q), 32)
    torch.cuda.synchronize()
    idx, sc = idx.cpu().numpy()[0], sc.cpu().numpy()[0]
    n_live = int(live.sum())
    assert set(idx[:n_live].tolist()) == set(np.nonzero(live)[0].tolist())
    assert np.all(idx[n_live:] == -1) and np.all(np.isneginf(sc[n_live:]))
