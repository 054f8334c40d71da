"""Pins of the Tensor Cache oracle ("Tensor Cache: Eviction-conditioned
Associative Memory for Transformers", gist.science, section "Metodologia")
(CPU)."""

import numpy as np
import torch

from oracle import tensor_cache as tc


def _tokens(n, d, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((n, d)).astype(np.float16), rng.standard_normal((n, d)).astype(np.float16),
            rng.standard_normal((3, d)).astype(np.float16))


def test_read_is_linear_attention_over_the_written_tokens():
    # the page's identity q (k outer v) = <q, k> v: after n writes the read
    # is the sum over the written tokens of eta lam^(n-1-t) <q, k_t> v_t
    d, n, lam, eta = 16, 40, 0.93, 0.25
    k, v, q = _tokens(n, d, 1)
    A = tc.write(np.zeros((d, d)), k, v, lam, eta)
    kk, vv, qq = (x.astype(np.float64) for x in (k, v, q))
    want = np.zeros((3, d))
    for t in range(n):
        w = eta * lam ** (n - 1 - t)
        for h in range(3):
            want[h] += w * float(qq[h] @ kk[t]) * vv[t]
    assert np.abs(tc.read(A, q) - want).max() < 1e-10 * max(1.0, np.abs(want).max())


def test_blocked_writes_equal_sequential_writes():
    # parallel weighted scan: a block of C tokens written at once as
    # A <- lam^C A + sum_c eta lam^(C-1-c) outer(k_c, v_c) equals C sequential
    # writes (the equivalence the page reports within fp32 epsilon)
    d, n, lam, eta = 8, 77, 0.97, 0.5
    k, v, _ = _tokens(n, d, 2)
    seq = tc.write(np.zeros((d, d)), k, v, lam, eta)
    A = np.zeros((d, d))
    kk, vv = k.astype(np.float64), v.astype(np.float64)
    for b0 in range(0, n, 32):
        blk = range(b0, min(n, b0 + 32))
        C = len(blk)
        A = lam ** C * A + sum(eta * lam ** (C - 1 - i) * np.outer(kk[t], vv[t]) for i, t in enumerate(blk))
    assert np.abs(A - seq).max() < 1e-12 * np.abs(seq).max()


def test_only_evicted_tokens_reach_the_matrix():
    d, W, hkv = 8, 5, 2
    rng = np.random.default_rng(3)
    c = tc.SeqLayerTC(hkv, d, W, 0.9, 0.3, 0.0)
    ks = rng.standard_normal((23, hkv, d)).astype(np.float16)
    vs = rng.standard_normal((23, hkv, d)).astype(np.float16)
    c.append(ks[:11], vs[:11])
    for t in range(11, 23):
        c.append(ks[t:t + 1], vs[t:t + 1])
    assert c.n_written == 23 - W and len(c.hot_k) == W
    for kv in range(hkv):
        want = tc.write(np.zeros((d, d)), ks[:23 - W, kv], vs[:23 - W, kv], 0.9, 0.3)
        assert np.abs(c.A[kv] - want).max() < 1e-12
    hk, _ = c.hot_arrays()
    assert np.array_equal(hk[:, :, :], ks[23 - W:].transpose(1, 0, 2))


def test_closed_gate_is_window_attention_and_the_read_adds_linearly():
    d, W, hkv, hq = 16, 7, 2, 4
    rng = np.random.default_rng(4)
    c = tc.SeqLayerTC(hkv, d, W, 0.95, 0.2, -1e9)
    c.append(rng.standard_normal((30, hkv, d)).astype(np.float16), rng.standard_normal((30, hkv, d)).astype(np.float16))
    q = rng.standard_normal((hq, d)).astype(np.float16)
    r = c.attend(q)
    hk, hv = c.hot_arrays()
    g = hq // hkv
    tq = torch.from_numpy(q.astype(np.float64)).view(hkv, g, 1, d)
    tk = torch.from_numpy(hk.astype(np.float64)).view(hkv, 1, W, d).expand(hkv, g, W, d)
    tv = torch.from_numpy(hv.astype(np.float64)).view(hkv, 1, W, d).expand(hkv, g, W, d)
    sdpa = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv).reshape(hq, d).numpy()
    assert np.abs(r["out"] - sdpa).max() < 1e-12  # sigmoid(-1e9) = 0: the window alone
    c.g = 0.0
    r2 = c.attend(q)
    assert np.abs(r2["out"] - (sdpa + 0.5 * r2["read"])).max() < 1e-12
    assert np.abs(r2["read"][0] - q[0].astype(np.float64) @ c.A[0]).max() < 1e-12
