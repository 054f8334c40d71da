"""Pins of the oracle's hot/cold paging simulator (CPU): brute-force
invariants and planted heavy hitters."""

import numpy as np
import pytest

from oracle import codec, params
from oracle.paging import SeqLayerCache

D, HKV, HQ, W = 16, 2, 4, 8


def _cache(tau=0.15, sticky=3, seed=0):
    return SeqLayerCache(HKV, D, W, codec.F3, params.rotation(D, seed), params.sketch(64, D, seed),
                         tau=tau, sticky=sticky)


def _tokens(rng, n):
    return (rng.standard_normal((n, HKV, D)).astype(np.float16),
            rng.standard_normal((n, HKV, D)).astype(np.float16))


def _check_invariants(c, after_append):
    hot_pos = c.hot_positions()
    live_pos = [p for p, l in zip(c.cold_pos, c.live) if l]
    assert len(set(hot_pos)) == len(hot_pos)
    assert set(hot_pos).isdisjoint(live_pos)
    assert set(hot_pos) | set(live_pos) == set(range(c.n_tokens))
    if after_append:
        assert len(c.hot) <= W
    for e in c.hot:
        if e.slot is not None:
            assert not c.live[e.slot] and c.cnt[e.slot] == 0
            assert c.cold_pos[e.slot] == e.pos
    n_tomb = sum(1 for l in c.live if not l)
    assert n_tomb == sum(1 for e in c.hot if e.slot is not None)


def test_prefill_splits_window_and_cold_in_order():
    rng = np.random.default_rng(0)
    c = _cache()
    k, v = _tokens(rng, 30)
    c.append(k, v)
    assert c.hot_positions() == list(range(22, 30))
    assert c.cold_pos == list(range(22))
    # cold slot j holds the quantised token j
    ref = codec.quantize(k[:22, 1], c.pi, c.s, c.fmt)
    got = c.cold_codes(1, "k")
    for key in ("a", "b", "signs", "R16", "rho16"):
        assert np.array_equal(got[key], ref[key])
    _check_invariants(c, True)


def test_random_walk_invariants():
    rng = np.random.default_rng(1)
    c = _cache(tau=0.05, sticky=1)
    for step in range(60):
        n = int(rng.integers(0, 6))
        k, v = _tokens(rng, n)
        c.append(k, v)
        _check_invariants(c, True)
        q = rng.standard_normal((HQ, D))
        live = [j for j, l in enumerate(c.live) if l]
        if live and rng.random() < 0.7:
            j = int(rng.choice(live))
            kk = c.cold_codes(0, "k")
            xh = codec.dequantize({kk_: kk[kk_][j:j + 1] for kk_ in kk}, c.pi, c.s, c.fmt)[0]
            q[:2] += 6.0 * xh / np.linalg.norm(xh) * np.sqrt(D)
        res = c.attend(q.astype(np.float16))
        c.promote(res["P"])
        _check_invariants(c, False)
        assert len(c.hot) <= W + HQ * int(1 / c.tau)
    assert c.n_promoted > 0 and c.n_evicted > 0


def _hitter_query(c, rng, slot, on):
    q = rng.standard_normal((HQ, D))
    if on:
        kk = c.cold_codes(0, "k")
        xh = codec.dequantize({k: kk[k][slot:slot + 1] for k in kk}, c.pi, c.s, c.fmt)[0]
        q[: HQ // HKV] += (np.log(len(c.live) + len(c.hot)) + 3.0) * np.sqrt(D) * xh / np.linalg.norm(xh) ** 2
    return q.astype(np.float16)


def test_sticky_promotion_fires_on_the_sticky_th_step():
    rng = np.random.default_rng(2)
    c = _cache(tau=0.15, sticky=3)
    k, v = _tokens(rng, 40)
    c.append(k, v)
    slot = 5
    on_steps = {1, 4, 5, 8, 9, 10}
    promoted_at = []
    for step in range(1, 14):
        kn, vn = _tokens(rng, 1)
        c.append(kn, vn)
        res = c.attend(_hitter_query(c, rng, slot, step in on_steps and c.live[slot]))
        if step in on_steps and c.live[slot]:
            assert res["P"][slot] > 2 * c.tau
        elif c.live[slot]:
            assert res["P"][slot] < c.tau / 2
        hits = c.promote(res["P"])
        if slot in hits:
            promoted_at.append(step)
    assert promoted_at == [10]
    # entered as the newest entry at step 10, three NEW tokens appended after it
    assert c.hot_tags()[-4] == slot and c.hot_positions()[-4] == 5
    assert not c.live[slot]
    assert not c.near_tau


def test_promoted_value_is_fp16_dequantisation_and_reeviction_revives_slot():
    rng = np.random.default_rng(3)
    c = _cache(tau=0.15, sticky=1)
    k, v = _tokens(rng, 200)  # long enough that no random token reaches tau
    c.append(k, v)
    slot = 7
    codes_before = c.cold_codes(1, "v")
    res = c.attend(_hitter_query(c, rng, slot, True))
    hits = c.promote(res["P"])
    assert hits[0] == slot  # the planted hitter has the largest P
    e = c.hot[W]
    ck = c.cold_codes(0, "k")
    xk = codec.dequantize({kk: ck[kk][slot:slot + 1] for kk in ck}, c.pi, c.s, c.fmt)[0]
    assert np.array_equal(e.k[0], xk.astype(np.float16))
    n_cold = len(c.live)
    # push W new tokens: the promoted entry is evicted without re-quantisation
    kn, vn = _tokens(rng, W)
    c.append(kn, vn)
    assert c.live[slot] and c.cnt[slot] == 0
    assert slot not in c.hot_tags()
    # the W older NEW entries were quantised; the promoted ones were revived
    assert len(c.live) == n_cold + W
    assert all(c.live[h] for h in hits)
    after = c.cold_codes(1, "v")
    for key in ("a", "b", "signs", "R16", "rho16"):
        assert np.array_equal(after[key][:n_cold], codes_before[key])
    _check_invariants(c, True)


def test_promotion_off_above_one():
    rng = np.random.default_rng(4)
    c = _cache(tau=2.0)
    k, v = _tokens(rng, 30)
    c.append(k, v)
    res = c.attend(_hitter_query(c, rng, 3, True))
    assert c.promote(res["P"]) == []
    assert all(t == -1 for t in c.hot_tags())


def test_evict_without_append_equals_the_append_path_eviction():
    """Evicting to a target after the tokens are in gives the same hot
    window, cold slots and codes as a window of that size during the append
    (the same FIFO step), and evicting to at least the hot count does
    nothing."""
    rng = np.random.default_rng(5)
    k, v = _tokens(rng, 30)
    a = _cache()  # window W = 8 during the append
    a.append(k, v)
    b = SeqLayerCache(HKV, D, 64, codec.F3, a.pi, a.s, tau=0.15, sticky=3)
    b.append(k, v)
    assert len(b.hot) == 30 and not b.live
    b.evict(40)
    assert len(b.hot) == 30 and not b.live
    b.evict(W)
    assert b.hot_positions() == a.hot_positions() and b.cold_pos == a.cold_pos
    assert b.n_evicted == a.n_evicted == 22
    for kv in range(HKV):
        for which in ("k", "v"):
            ga, gb = a.cold_codes(kv, which), b.cold_codes(kv, which)
            for key in ("a", "b", "signs", "R16", "rho16"):
                assert np.array_equal(ga[key], gb[key])
    b.evict(0)
    assert not b.hot and b.cold_pos == list(range(30))


def test_evict_revives_a_promoted_entry():
    rng = np.random.default_rng(6)
    c = _cache(tau=0.15, sticky=1)
    k, v = _tokens(rng, 200)
    c.append(k, v)
    slot = 11
    res = c.attend(_hitter_query(c, rng, slot, True))
    hits = c.promote(res["P"])
    assert slot in hits and slot in c.hot_tags()
    n_cold = len(c.live)
    c.evict(0)  # every hot entry leaves: the W NEW ones are quantised, the promoted ones revived
    assert not c.hot and c.live[slot] and c.cnt[slot] == 0
    assert len(c.live) == n_cold + W and all(c.live)
    _check_invariants(c, True)
