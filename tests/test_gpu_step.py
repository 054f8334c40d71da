"""GPU parity of tq_decode_step (one call per layer and decode step: append,
then attention, with the query preparation inside the append's launch).

Against the oracle: outputs within 2e-3 max-abs, codes, hot FIFO, tombstones
and sticky counters as in the other paging tests.  Against the separate calls
(tq_quantize_append, then tq_decode_attention) on a second cache built from
the same seed: outputs and exported state equal bit for bit, since the step
prepares the queries with the same arithmetic in the same order."""

import numpy as np
import pytest

from compressed_kv_decode_amd import workloads as wl

from gpu_helpers import dev, make_cache
from test_gpu_parity import _run_paging

pytestmark = pytest.mark.gpu


def test_decode_step_tinyllama_deferred_promotion_against_oracle():
    """TinyLlama shape (32 q / 4 kv: groups of 8, d 64) with planted heavy
    hitters; two layers, deferred promotion: each step's launch runs the
    append, the other layer's promotion and the query preparation."""
    w = wl.make("tinyllama").with_(steps=20)
    r = _run_paging(w, [0, 7], w.steps, check_every=5, deferred=True, step_call=True)
    print("decode step, tinyllama:", r)
    assert r["promoted"] >= 2


@pytest.mark.parametrize("fmt", [wl.F3, wl.F4])
def test_decode_step_llama8b_slice_against_oracle(fmt):
    """Llama-3.1-8B heads (32 q / 8 kv, d 128) on two sequences of a shorter
    context (several tiles, ragged tails)."""
    w = wl.make("llama8b", fmt=fmt).with_(n_seq=2, n_layers=1, prefill=(3000, 1337), formats=(fmt,), steps=3)
    r = _run_paging(w, [0], w.steps, step_call=True)
    print("decode step, llama8b slice", fmt, r)


def _state(cache, seq, layer):
    tags, hk, hv = cache.export_hot(seq, layer)
    live, stk = cache.export_paging(seq, layer, cache.max_context)
    return (np.array(tags), hk, hv), (live, stk), cache.stats(seq, layer)


@pytest.mark.parametrize("d,hq,hkv,fmt", [(64, 4, 4, wl.F3), (64, 4, 2, wl.F25), (128, 32, 8, wl.F3),
                                          (128, 8, 1, wl.F4), (128, 16, 16, wl.F3)])
def test_decode_step_equals_separate_calls(d, hq, hkv, fmt):
    """Groups of 1, 2, 4 and 8 query heads, both head dims: the step call and
    the separate calls give equal outputs and state on every step, with two
    layers and deferred promotion, and with one step whose append is large
    (40 tokens: no query preparation in the append launch)."""
    import torch
    w = wl.make("tiny").with_(head_dim=d, n_q_heads=hq, n_kv_heads=hkv, formats=(fmt, fmt), n_layers=2, n_seq=3,
                               prefill=(900, 333, 64), window=64, steps=4, outlier_channels=2, tau=0.05, sticky=1)
    seqs = [0, 1, 2]
    a, b = make_cache(w, max_context=1024), make_cache(w, max_context=1024)
    for c in (a, b):
        for l in range(2):
            ks, vs = zip(*[wl.prefill_kv(w, l, sq) for sq in seqs])
            c.append(l, seqs, [w.prefill[sq] for sq in seqs], dev(np.concatenate(ks)), dev(np.concatenate(vs)))
    rng = np.random.default_rng(7)
    for step in range(w.steps):
        n_new = [40, 1, 3] if step == 2 else [1, 1, 1]
        for l in range(2):
            k = (rng.standard_normal((sum(n_new), hkv, d)) * 0.5).astype(np.float16)
            v = (rng.standard_normal((sum(n_new), hkv, d)) * 0.5).astype(np.float16)
            q = rng.standard_normal((len(seqs), hq, d)).astype(np.float16)
            a.append(l, seqs, n_new, dev(k), dev(v))
            oa = a.attend(l, seqs, dev(q))
            a.promote(l, seqs, deferred=True)
            ob = b.step(l, seqs, n_new, dev(k), dev(v), dev(q))
            b.promote(l, seqs, deferred=True)
            torch.cuda.synchronize()
            assert torch.equal(oa, ob), f"step {step} layer {l}: outputs differ"
    a.flush()
    b.flush()
    torch.cuda.synchronize()
    for l in range(2):
        for sq in seqs:
            ta, pa, sa = _state(a, sq, l)
            tb, pb, sb = _state(b, sq, l)
            for x, y in zip(ta, tb):
                assert np.array_equal(x, y), f"seq {sq} layer {l}: hot window differs"
            for x, y in zip(pa, pb):
                assert np.array_equal(x, y), f"seq {sq} layer {l}: paging state differs"
            assert sa == sb and sa["status"] == 0 and sa["device_error"] == 0
            for kv in (0, 1) if sa["cold_len"] > 0 else ():
                for h in range(hkv):
                    ca = a.export_codes(sq, l, h, kv, 0, sa["cold_len"])
                    cb = b.export_codes(sq, l, h, kv, 0, sb["cold_len"])
                    assert np.array_equal(ca, cb), f"seq {sq} layer {l} kv head {h}: codes differ"


def test_decode_step_tensor_cache_tier_equals_separate_calls():
    """With the Tensor Cache cold tier the append takes the general path
    (no query preparation in its launch): the step call still equals the
    separate calls bit for bit, outputs and matrices."""
    import torch
    from compressed_kv_decode_amd import tqkv
    w = wl.make("tiny").with_(n_seq=2, prefill=(500, 130), window=64, steps=3)
    seqs = [0, 1]
    caches = [tqkv.Cache(n_seq_max=2, n_layers=1, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads,
                         head_dim=w.head_dim, hot_window=w.window, max_context=1024, formats=[w.formats[0]],
                         seed=w.seed, cold_tier=tqkv.COLD_TENSOR_CACHE, tc_lambda=0.99, tc_eta=0.5, tc_gate=0.3)
              for _ in range(2)]
    a, b = caches
    ks, vs = zip(*[wl.prefill_kv(w, 0, sq) for sq in seqs])
    for c in caches:
        c.append(0, seqs, [w.prefill[sq] for sq in seqs], dev(np.concatenate(ks)), dev(np.concatenate(vs)))
    rng = np.random.default_rng(11)
    for step in range(w.steps):
        k = rng.standard_normal((2, w.n_kv_heads, w.head_dim)).astype(np.float16)
        v = rng.standard_normal((2, w.n_kv_heads, w.head_dim)).astype(np.float16)
        q = rng.standard_normal((2, w.n_q_heads, w.head_dim)).astype(np.float16)
        a.append(0, seqs, [1, 1], dev(k), dev(v))
        oa = a.attend(0, seqs, dev(q))
        ob = b.step(0, seqs, [1, 1], dev(k), dev(v), dev(q))
        torch.cuda.synchronize()
        assert torch.equal(oa, ob), f"step {step}: outputs differ"
    for sq in seqs:
        for h in range(w.n_kv_heads):
            assert np.array_equal(a.export_tensor_cache(sq, 0, h), b.export_tensor_cache(sq, 0, h))


def test_decode_step_more_sequences_than_one_launch_batch():
    """130 sequences: the appends and the attention run in two launch batches
    (at most 128 sequences each), so the step call prepares the queries in the
    attention's own launches; results equal the separate calls bit for bit."""
    import torch
    n = 130
    w = wl.make("tiny").with_(n_seq=n, n_q_heads=4, n_kv_heads=2, head_dim=64, window=64,
                               prefill=tuple(100 + (i % 7) * 9 for i in range(n)), steps=2)
    seqs = list(range(n))
    a, b = make_cache(w, max_context=256), make_cache(w, max_context=256)
    ks, vs = zip(*[wl.prefill_kv(w, 0, sq) for sq in seqs])
    for c in (a, b):
        c.append(0, seqs, [w.prefill[sq] for sq in seqs], dev(np.concatenate(ks)), dev(np.concatenate(vs)))
    rng = np.random.default_rng(5)
    for step in range(w.steps):
        k = rng.standard_normal((n, 2, 64)).astype(np.float16)
        v = rng.standard_normal((n, 2, 64)).astype(np.float16)
        q = rng.standard_normal((n, 4, 64)).astype(np.float16)
        a.append(0, seqs, [1] * n, dev(k), dev(v))
        oa = a.attend(0, seqs, dev(q))
        ob = b.step(0, seqs, [1] * n, dev(k), dev(v), dev(q))
        torch.cuda.synchronize()
        assert torch.equal(oa, ob), f"step {step}: outputs differ"
        assert torch.isfinite(ob).all()
