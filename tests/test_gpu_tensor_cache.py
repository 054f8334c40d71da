"""The Tensor Cache cold tier on the GPU against the oracle ("Tensor Cache:
Eviction-conditioned Associative Memory for Transformers", gist.science,
section "Metodologia"): the matrices A written by evictions (prefill rows
that leave at once, ring entries pushed out by decode steps or by tq_evict)
and the merged outputs y_local + sigmoid(g) q A."""

import numpy as np
import pytest

from compressed_kv_decode_amd import tqkv
from compressed_kv_decode_amd import workloads as wl
from oracle import tensor_cache as tc

from gpu_helpers import assert_out_close, dev

pytestmark = pytest.mark.gpu

A_RTOL = 1e-4  # fp32 blocked accumulation against fp64 sequential writes, relative to max |A|


def _sync():
    import torch
    torch.cuda.synchronize()


def _f32(*xs):
    """The configuration carries lambda, eta and g as fp32: the oracle gets
    the same values (lambda^n over thousands of tokens tells them apart)."""
    return tuple(float(np.float32(x)) for x in xs)


def _cache(w, lam, eta, g, max_context=None):
    return tqkv.Cache(n_seq_max=w.n_seq, n_layers=1, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads,
                      head_dim=w.head_dim, hot_window=w.window, max_context=max_context or w.max_context(),
                      formats=[w.formats[0]], seed=w.seed, cold_tier=tqkv.COLD_TENSOR_CACHE, tc_lambda=lam,
                      tc_eta=eta, tc_gate=g)


def _check_state(cache, oc, seq_ids, what):
    for sq in seq_ids:
        for kvh in range(oc[sq].hkv):
            got = cache.export_tensor_cache(sq, 0, kvh).astype(np.float64)
            want = oc[sq].A[kvh]
            scale = max(1e-30, np.abs(want).max())
            err = np.abs(got - want).max() / scale
            assert err <= A_RTOL, f"{what} seq {sq} kvh {kvh}: A rel err {err:.2e}"
        st = cache.stats(sq, 0)
        assert st["status"] == 0 and st["cold_len"] == 0 and st["hot_len"] == len(oc[sq].hot_k)


def _attend(cache, oc, w, seq_ids, step, what):
    q = np.stack([wl.query(w, 0, sq, step) for sq in seq_ids])
    out = cache.attend(0, seq_ids, dev(q)).cpu().numpy()
    for i, sq in enumerate(seq_ids):
        res = oc[sq].attend(q[i])
        assert_out_close(out[i], res["out"], f"{what} seq {sq}")
        assert np.abs(res["read"]).max() > 1e-2  # the second level contributes


@pytest.mark.parametrize("shape", ["tiny", "llama8b"])
def test_tensor_cache_tier_against_oracle(shape):
    if shape == "tiny":
        w = wl.make("tiny").with_(n_seq=1, window=64, prefill=(300,), steps=12)
        lam, eta, g = _f32(0.99, 0.05, 0.3)
    else:
        w = wl.make("llama8b").with_(n_seq=2, n_layers=1, prefill=(3000, 1337), formats=(wl.F3,), steps=12)
        lam, eta, g = _f32(0.999, 1.0 / 128, 0.0)
    seq_ids = list(range(w.n_seq))
    cache = _cache(w, lam, eta, g)
    oc = {sq: tc.SeqLayerTC(w.n_kv_heads, w.head_dim, w.window, lam, eta, g) for sq in seq_ids}
    ks, vs = zip(*[wl.prefill_kv(w, 0, sq) for sq in seq_ids])
    cache.append(0, seq_ids, list(w.prefill), dev(np.concatenate(ks)), dev(np.concatenate(vs)))
    for i, sq in enumerate(seq_ids):
        oc[sq].append(ks[i], vs[i])
    _sync()
    _check_state(cache, oc, seq_ids, "prefill")
    for step in range(w.steps):
        sk, sv = zip(*[wl.step_kv(w, 0, sq, step) for sq in seq_ids])
        cache.append(0, seq_ids, [1] * len(seq_ids), dev(np.concatenate(sk)), dev(np.concatenate(sv)))
        for i, sq in enumerate(seq_ids):
            oc[sq].append(sk[i], sv[i])
        _attend(cache, oc, w, seq_ids, step, f"{shape} step {step}")
        if step % 4 == 3:
            _sync()
            _check_state(cache, oc, seq_ids, f"{shape} step {step}")


@pytest.mark.parametrize("d,lam", [(64, 0.9), (128, 0.9995)])
def test_tensor_cache_large_appends_in_segments(d, lam):
    """Appends of 512 or more new tokens take the segmented MFMA write: a
    second large append evicts the ring's entries first, then input rows;
    ragged sequences give different segment counts (lambda 0.9 drives old
    weights below fp32's range, as the sequential writes do)."""
    w = wl.make("tiny").with_(head_dim=d, n_seq=3, window=64, prefill=(200, 90, 600), steps=1)
    lam, eta, g = _f32(lam, 0.02, 0.1)
    seq_ids = [0, 1, 2]
    cache = _cache(w, lam, eta, g, max_context=20000)
    oc = {sq: tc.SeqLayerTC(w.n_kv_heads, w.head_dim, w.window, lam, eta, g) for sq in seq_ids}
    ks, vs = zip(*[wl.prefill_kv(w, 0, sq) for sq in seq_ids])
    cache.append(0, seq_ids, list(w.prefill), dev(np.concatenate(ks)), dev(np.concatenate(vs)))
    for i, sq in enumerate(seq_ids):
        oc[sq].append(ks[i], vs[i])
    _sync()
    _check_state(cache, oc, seq_ids, "first append")
    rng = np.random.default_rng(77)
    n2 = [5000, 700, 0]
    k2 = [rng.standard_normal((n, w.n_kv_heads, d)).astype(np.float16) for n in n2]
    v2 = [rng.standard_normal((n, w.n_kv_heads, d)).astype(np.float16) for n in n2]
    cache.append(0, seq_ids, n2, dev(np.concatenate(k2)), dev(np.concatenate(v2)))
    for i, sq in enumerate(seq_ids):
        if n2[i]:
            oc[sq].append(k2[i], v2[i])
    _sync()
    _check_state(cache, oc, seq_ids, "second append")
    _attend(cache, oc, w, seq_ids, 0, f"d {d} after large appends")


def test_tensor_cache_evict_without_append():
    """tq_evict in the tensor-cache tier writes the ring entries it pushes out."""
    w = wl.make("tiny").with_(n_seq=2, window=64, prefill=(200, 90), steps=2)
    lam, eta, g = _f32(0.97, 0.1, -0.5)
    seq_ids = [0, 1]
    cache = _cache(w, lam, eta, g)
    oc = {sq: tc.SeqLayerTC(w.n_kv_heads, w.head_dim, w.window, lam, eta, g) for sq in seq_ids}
    ks, vs = zip(*[wl.prefill_kv(w, 0, sq) for sq in seq_ids])
    cache.append(0, seq_ids, list(w.prefill), dev(np.concatenate(ks)), dev(np.concatenate(vs)))
    for i, sq in enumerate(seq_ids):
        oc[sq].append(ks[i], vs[i])
    for target in (40, 5, 0):
        cache.evict(0, seq_ids, target)
        for sq in seq_ids:
            o = oc[sq]
            while len(o.hot_k) > target:
                k, v = o.hot_k.pop(0), o.hot_v.pop(0)
                for kv in range(o.hkv):
                    o.A[kv] = tc.write(o.A[kv], k[kv][None], v[kv][None], lam, eta)
        _sync()
        _check_state(cache, oc, seq_ids, f"evict to {target}")
    _attend(cache, oc, w, seq_ids, 0, "after evicting everything")
