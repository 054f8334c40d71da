"""GPU parity: the HIP path through the C ABI against the oracle on the same
seeded inputs.  Codes bit-exact outside the 1e-6 boundary band, logits within
1e-3 relative (of max(|l|, 1)), outputs within 2e-3 max-abs in fp32."""

import numpy as np
import pytest

from compressed_kv_decode_amd import workloads as wl
from oracle import attention, codec, params
from oracle.paging import SeqLayerCache

from gpu_helpers import (assert_adoption, assert_logits_close, assert_out_close, check_codes, dev, fmt_of, make_cache,
                         oracle_params)

pytestmark = pytest.mark.gpu


def _sync():
    import torch
    torch.cuda.synchronize()


def test_rotation_and_sketch_match_oracle():
    for d in (64, 128):
        w = wl.make("tiny").with_(head_dim=d, seed=7)
        c = make_cache(w)
        pi, s = c.rotation()
        assert np.abs(pi.astype(np.float64) - params.rotation(d, 7)).max() < 1e-6
        assert np.abs(s.astype(np.float64) - params.sketch(64, d, 7)).max() < 1e-6
        c = make_cache(w, rotation_kind=1)
        pi, s = c.rotation()
        assert np.abs(pi.astype(np.float64) - params.hadamard_rotation(d, 7)).max() < 1e-7
        assert np.abs(s.astype(np.float64) - params.sketch(64, d, 7)).max() < 1e-6


def _oracle_sync_codes(oc, cache, seq, layer, what):
    """Compare every cold slot's codes with the oracle simulator's; adopt the
    GPU's alternative where (and only where) the boundary band allows it."""
    n = len(oc.live)
    adopted = 0
    for kvh in range(oc.hkv):
        for kv, lst, bands in ((0, oc.cold_k[kvh], oc.band_k[kvh]), (1, oc.cold_v[kvh], oc.band_v[kvh])):
            if n == 0:
                continue
            g = cache.export_codes(seq, layer, kvh, kv, 0, n)
            stack = {k: np.stack([c[k] for c in lst]) for k in ("a", "b", "R16", "rho16", "signs")}
            orec = codec.pack_records(stack, oc.d, oc.fmt)
            for i in np.nonzero(np.any(g != orec, axis=1))[0]:
                gc = codec.unpack_records(g[i:i + 1], oc.d, oc.fmt)
                b = bands[i]
                pb = (gc["a"][0] != lst[i]["a"]) | (gc["b"][0] != lst[i]["b"])
                assert not np.any(pb & ~b["pair"]), f"{what}: slot {i} kv{kv} head {kvh} pair codes"
                assert gc["R16"][0] == lst[i]["R16"] or b["R"], f"{what}: slot {i} R"
                assert gc["rho16"][0] == lst[i]["rho16"] or b["rho"], f"{what}: slot {i} rho"
                assert not np.any((gc["signs"][0] != lst[i]["signs"]) & ~b["sign"]), f"{what}: slot {i} signs"
                lst[i] = {k: gc[k][0] for k in ("a", "b", "R16", "rho16", "signs")}
                adopted += 1
    return adopted


def _check_hot(oc, cache, seq, layer, what):
    tags, hk, hv = cache.export_hot(seq, layer)
    assert tags == oc.hot_tags(), f"{what}: hot FIFO tags differ"
    ok, ov = oc.hot_arrays()
    # NEW entries are exact copies; promoted ones are fp16 roundings of a
    # dequantisation computed in fp32 on the GPU and fp64 in the oracle: one
    # fp16 ulp plus the fp32 absolute error of a length-d dot product
    for e_i, t in enumerate(tags):
        a, b = hk[:, e_i].astype(np.float64), ok[:, e_i].astype(np.float64)
        c, d = hv[:, e_i].astype(np.float64), ov[:, e_i].astype(np.float64)
        if t < 0:
            assert np.array_equal(a, b) and np.array_equal(c, d), f"{what}: NEW hot entry {e_i}"
        else:
            for got, want, name in ((a, b, "key"), (c, d, "value")):
                tol = 2.0 ** -10 * np.abs(want) + 2e-6 * np.abs(want).max(axis=1, keepdims=True)
                assert np.all(np.abs(got - want) <= tol), f"{what}: promoted {name} {e_i}"


def _check_paging(oc, cache, seq, layer, what):
    n = len(oc.live)
    live, stk = cache.export_paging(seq, layer, n)
    assert np.array_equal(live, np.array(oc.live, dtype=bool)), f"{what}: tombstones differ"
    assert np.array_equal(stk, np.array(oc.cnt)), f"{what}: sticky counters differ"


GATE_BAND = 1e-4  # a group whose best hot logit is this close to the threshold may be decided either way


def _attend_and_compare(oc, cache, w, layer, seq_ids, qs, what, gate=None):
    """One attention step for the sequences in seq_ids (oracle per sequence;
    gate: the hot-first threshold, or None for the plain step)."""
    import torch
    q = np.stack(qs)
    logits = torch.full((len(seq_ids), w.n_q_heads, cache.logits_stride), float("nan"), device="cuda")
    out = cache.attend(layer, seq_ids, dev(q), logits=logits, gate=gate)
    _sync()
    out, logits = out.cpu().numpy(), logits.cpu().numpy()
    res_all = []
    for i, s in enumerate(seq_ids):
        res = oc[s].attend(q[i], gate=np.inf if gate is None else gate)
        if gate is not None:
            assert np.all(np.abs(res["gate_margin"]) > GATE_BAND), f"{what}: a group sits on the threshold"
        nh = len(oc[s].hot)
        want_hot = np.full((w.n_q_heads, cache.hot_capacity), -np.inf)
        want_hot[:, :nh] = res["logits_hot"]
        assert_logits_close(logits[i, :, :cache.hot_capacity], want_hot, f"{what} seq {s} hot")
        nc = len(oc[s].live)
        want_cold = np.full((w.n_q_heads, cache.logits_stride - cache.hot_capacity), -np.inf)
        want_cold[:, :nc] = res["logits_cold"]
        assert_logits_close(logits[i, :, cache.hot_capacity:], want_cold, f"{what} seq {s} cold")
        assert_out_close(out[i], res["out"], f"{what} seq {s} out")
        res_all.append(res)
    return res_all


def _run_paging(w, layers, steps, seq_ids=None, check_every=1, keep=False, gate=None, rotation_kind=0,
                deferred=False, step_call=False):
    """Prefill + decode steps (append, attend, promote) against the oracle
    (keep: also return the cache and the oracle simulators; rotation_kind 1:
    both sides rotate with the randomized Hadamard matrix; deferred: promote
    with tq_promote_deferred, so that each promotion runs in the next layer's
    append launch unless a check between them launches it first; step_call:
    each step's append and attention are one tq_decode_step call, whose
    outputs are compared, the logits being checked by the other tests)."""
    seq_ids = list(range(w.n_seq)) if seq_ids is None else seq_ids
    cache = make_cache(w, rotation_kind=rotation_kind)
    fm = [fmt_of(f) for f in w.formats]
    pi, s = oracle_params(w, rotation_kind)
    oc = {(l, sq): SeqLayerCache(w.n_kv_heads, w.head_dim, w.window, fm[l], pi, s, tau=w.tau, sticky=w.sticky,
                                 v_qjl=w.v_qjl) for l in layers for sq in seq_ids}
    adopted = 0
    for l in layers:
        ks, vs = zip(*[wl.prefill_kv(w, l, sq) for sq in seq_ids])
        cache.append(l, seq_ids, [w.prefill[sq] for sq in seq_ids], dev(np.concatenate(ks)), dev(np.concatenate(vs)))
        for i, sq in enumerate(seq_ids):
            oc[(l, sq)].append(ks[i], vs[i])
        _sync()
        for sq in seq_ids:
            adopted += _oracle_sync_codes(oc[(l, sq)], cache, sq, l, f"prefill l{l} s{sq}")
            _check_hot(oc[(l, sq)], cache, sq, l, f"prefill l{l} s{sq}")
    promoted = 0
    for step in range(steps):
        for l in layers:
            ks, vs = zip(*[wl.step_kv(w, l, sq, step) for sq in seq_ids])
            qs = [wl.query(w, l, sq, step) for sq in seq_ids]
            if step_call:
                out = cache.step(l, seq_ids, [1] * len(seq_ids), dev(np.concatenate(ks)), dev(np.concatenate(vs)),
                                 dev(np.stack(qs)))
            else:
                cache.append(l, seq_ids, [1] * len(seq_ids), dev(np.concatenate(ks)), dev(np.concatenate(vs)))
            for i, sq in enumerate(seq_ids):
                oc[(l, sq)].append(ks[i], vs[i])
            _sync()
            for sq in seq_ids:
                adopted += _oracle_sync_codes(oc[(l, sq)], cache, sq, l, f"step {step} l{l} s{sq}")
            view = {sq: oc[(l, sq)] for sq in seq_ids}
            if step_call:
                out = out.cpu().numpy()
                res = [view[sq].attend(qs[i]) for i, sq in enumerate(seq_ids)]
                for i, sq in enumerate(seq_ids):
                    assert_out_close(out[i], res[i]["out"], f"step {step} l{l} seq {sq} out (decode step call)")
            else:
                res = _attend_and_compare(view, cache, w, l, seq_ids, qs, f"step {step} l{l}", gate=gate)
            cache.promote(l, seq_ids, deferred=deferred)
            for i, sq in enumerate(seq_ids):
                promoted += len(oc[(l, sq)].promote(res[i]["P"]))
            _sync()
            if step % check_every == 0 or step == steps - 1:
                for sq in seq_ids:
                    _check_hot(oc[(l, sq)], cache, sq, l, f"step {step} l{l} s{sq}")
                    _check_paging(oc[(l, sq)], cache, sq, l, f"step {step} l{l} s{sq}")
                    st = cache.stats(sq, l)
                    assert st["status"] == 0 and st["device_error"] == 0
                    assert st["cold_len"] == len(oc[(l, sq)].live)
                    assert st["hot_len"] == len(oc[(l, sq)].hot)
    near = sum(len(o.near_tau) for o in oc.values())
    checked = sum(len(o.live) * o.hkv * 2 for o in oc.values())  # every cold record ever written, K and V
    assert_adoption(adopted, checked, f"{w.name} layers {layers}")
    r = dict(adopted=adopted, checked=checked, promoted=promoted, near_tau=near)
    return (r, cache, oc) if keep else r


def test_tiny_workload_full():
    """1 seq, 1 layer, 4 heads, d 64, 1024 prefill (768 cold F3), 8 steps."""
    w = wl.make("tiny")
    r = _run_paging(w, [0], w.steps)
    print("tiny:", r)


def test_tinyllama_paging_with_promotion():
    """TinyLlama-shaped attention (32 q / 4 kv, d 64, 512 hot + 1024 cold F3)
    with planted heavy hitters; two of the 22 layers, all 50 steps."""
    w = wl.make("tinyllama")
    r = _run_paging(w, [0, 7], w.steps)
    print("tinyllama:", r)
    assert r["promoted"] >= 2
    assert r["near_tau"] == 0


@pytest.mark.parametrize("layers", [[0, 7], [0]])
def test_deferred_promotion_matches_the_oracle(layers):
    """tq_promote_deferred on the TinyLlama shape with planted heavy hitters:
    with two layers each promotion runs inside the other layer's next small
    append (no call in between launches it); with one layer the next append
    is of the same layer and launches it first.  Hot FIFO, tombstones, sticky
    counters and outputs against the oracle, which promotes at once."""
    w = wl.make("tinyllama").with_(steps=30)
    r = _run_paging(w, layers, w.steps, check_every=1000, deferred=True)
    print("deferred promotion", layers, r)
    assert r["promoted"] >= 2
    assert r["near_tau"] == 0


def test_evict_without_append():
    """tq_evict after decode steps with promotions: down to fewer hot entries
    (NEW ones quantised into cold slots, PROMOTED ones reviving theirs), then
    to none; codes, hot FIFO, tombstones, sticky counters and attention
    against the oracle after each."""
    w = wl.make("tinyllama").with_(steps=16)
    r, cache, oc = _run_paging(w, [0], w.steps, keep=True)
    assert r["promoted"] >= 1
    seq_ids = list(range(w.n_seq))
    for i, target in enumerate((w.window - 37, w.window + 50, 3, 0)):
        cache.evict(0, seq_ids, target)
        for sq in seq_ids:
            oc[(0, sq)].evict(target)
        _sync()
        for sq in seq_ids:
            what = f"evict to {target} s{sq}"
            _oracle_sync_codes(oc[(0, sq)], cache, sq, 0, what)
            _check_hot(oc[(0, sq)], cache, sq, 0, what)
            _check_paging(oc[(0, sq)], cache, sq, 0, what)
            st = cache.stats(sq, 0)
            assert st["status"] == 0 and st["device_error"] == 0
            assert st["hot_len"] == len(oc[(0, sq)].hot) and st["cold_len"] == len(oc[(0, sq)].live)
        view = {sq: oc[(0, sq)] for sq in seq_ids}
        qs = [wl.query(w, 0, sq, w.steps + i) for sq in seq_ids]
        res = _attend_and_compare(view, cache, w, 0, seq_ids, qs, f"after evict to {target}")
        cache.promote(0, seq_ids)  # the step's promotion keeps the counters of both sides in step
        for j, sq in enumerate(seq_ids):
            oc[(0, sq)].promote(res[j]["P"])


@pytest.mark.parametrize("fmt", [wl.F3, wl.F4, wl.F25])
def test_llama8b_shaped_slice(fmt):
    """Llama-3.1-8B-shaped heads (32 q / 8 kv, d 128) on one layer of two
    sequences with a shorter context (several tiles and a ragged tail)."""
    w = wl.make("llama8b", fmt=fmt).with_(n_seq=2, n_layers=1, prefill=(3000, 1337), formats=(fmt,), steps=3)
    r = _run_paging(w, [0], w.steps)
    print("llama8b slice", fmt, r)


@pytest.mark.parametrize("fmt", [wl.F3, wl.F4])
def test_hadamard_rotation_llama8b_slice(fmt):
    """The randomized Hadamard rotation in place of the Haar one: codes,
    logits, outputs and paging against the oracle rotated the same way."""
    w = wl.make("llama8b", fmt=fmt).with_(n_seq=2, n_layers=1, prefill=(2500, 900), formats=(fmt,), steps=3)
    r = _run_paging(w, [0], w.steps, rotation_kind=1)
    print("llama8b slice, Hadamard rotation", fmt, r)


def test_ragged_mixed_formats_slice():
    """Mistral-shaped ragged batch: 5 sequences of different lengths, F3 and
    F4 layers, eviction + promotion with heavy hitters."""
    w = wl.make("ragged").with_(n_seq=5, n_layers=2, prefill=(1024, 1500, 2100, 777 + 512, 4000), steps=6,
                                formats=(wl.F3, wl.F4))
    r = _run_paging(w, [0, 1], w.steps, check_every=2)
    print("ragged slice:", r)


def test_group_sizes_and_head_dims():
    for d, hq, hkv, fmt in [(64, 2, 2, wl.F4), (64, 4, 2, wl.F25), (128, 8, 1, wl.F3), (128, 16, 2, (2, 3, 64))]:
        w = wl.make("tiny").with_(head_dim=d, n_q_heads=hq, n_kv_heads=hkv, formats=(fmt,), prefill=(700,),
                                   window=64, steps=2, outlier_channels=2)
        _run_paging(w, [0], w.steps)


def test_short_context_and_empty_appends():
    """Context shorter than the window (no cold tokens), an empty append and
    sequence ids that are not contiguous."""
    import torch
    w = wl.make("tiny").with_(n_seq=3, prefill=(100, 300, 40), steps=0)
    cache = make_cache(w, n_seq_max=6)
    pi, s = oracle_params(w)
    k, v = wl.prefill_kv(w, 0, 0)
    cache.append(0, [4], [100], dev(k), dev(v))
    cache.append(0, [4], [0], None, None)
    oc = SeqLayerCache(4, 64, w.window, fmt_of(wl.F3), pi, s)
    oc.append(k, v)
    _sync()
    st = cache.stats(4, 0)
    assert st["cold_len"] == 0 and st["hot_len"] == 100
    q = wl.query(w, 0, 0, 0)
    out = cache.attend(0, [4], dev(q[None])).cpu().numpy()
    res = oc.attend(q)
    assert_out_close(out[0], res["out"], "short context")
    # never-written sequence: attention over nothing gives zeros
    out2 = cache.attend(0, [1], dev(q[None])).cpu().numpy()
    assert np.all(out2 == 0.0)


def test_large_appends_that_split_tiles():
    """Several large appends per sequence, two sequences per call, so the
    quantiser's items start and end in the middle of cold tiles (value tiles
    are OR-ed into earlier bits, codes of slots outside the launch masked).
    Every cold record of every kv head, K and V, against the oracle's codes
    of the same evicted fp16 vectors, for the three code layouts."""
    rng = np.random.default_rng(11)
    W = 64
    sizes = [(100, 70), (45, 9), (77, 130), (9, 33), (200, 64)]  # every call has more than 8 new tokens
    for d, fmt in [(128, wl.F3), (128, wl.F4), (64, wl.F25)]:
        w = wl.make("tiny").with_(head_dim=d, n_q_heads=4, n_kv_heads=2, formats=(fmt,), window=W, n_seq=2,
                                  prefill=(431, 306), steps=0)
        cache = make_cache(w, n_seq_max=2, max_context=1024)
        pi, s = oracle_params(w)
        adopted = checked = 0
        scale = np.ones(d, dtype=np.float32)
        scale[rng.choice(d, 3, replace=False)] = 8.0  # outlier channels
        ks, vs = [[], []], [[], []]
        for n in sizes:
            kk = [(rng.standard_normal((m, 2, d)) * scale).astype(np.float16) for m in n]
            vv = [(rng.standard_normal((m, 2, d)) * scale).astype(np.float16) for m in n]
            cache.append(0, [0, 1], list(n), dev(np.concatenate(kk)), dev(np.concatenate(vv)))
            for i in range(2):
                ks[i].append(kk[i])
                vs[i].append(vv[i])
        _sync()
        for i in range(2):
            K, V = np.concatenate(ks[i]), np.concatenate(vs[i])
            ncold = K.shape[0] - W
            assert cache.stats(i, 0)["cold_len"] == ncold
            for h in range(2):
                for kv, X in ((0, K), (1, V)):
                    rec = cache.export_codes(i, 0, h, kv, 0, ncold)
                    _, nd, nb = check_codes(rec, X[:ncold, h, :], pi, s, fmt_of(fmt), d,
                                            f"d {d} {fmt} seq {i} kv head {h} {'KV'[kv]}")
                    adopted += nd
                    checked += ncold
        assert_adoption(adopted, checked, f"large appends d {d} {fmt}")


def test_deterministic_rerun():
    import torch
    w = wl.make("llama8b").with_(n_seq=2, n_layers=1, prefill=(2500, 999), formats=(wl.F4,), steps=1)
    outs = []
    for _ in range(2):
        cache = make_cache(w)
        ks, vs = zip(*[wl.prefill_kv(w, 0, sq) for sq in range(2)])
        cache.append(0, [0, 1], list(w.prefill), dev(np.concatenate(ks)), dev(np.concatenate(vs)))
        q = np.stack([wl.query(w, 0, sq, 0) for sq in range(2)])
        o = cache.attend(0, [0, 1], dev(q)).cpu().numpy()
        recs = cache.export_codes(1, 0, 3, 1, 0, 487)
        outs.append((o, recs))
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1], outs[1][1])


def test_import_export_round_trip_and_decode_on_oracle_codes():
    """Oracle codes imported through the ABI decode to the oracle's attention:
    the decode kernel checked on its own, independent of the quantiser."""
    w = wl.make("llama8b").with_(n_seq=1, n_layers=1, prefill=(1800,), formats=(wl.F3,), steps=0)
    cache = make_cache(w)
    pi, s = oracle_params(w)
    fm = fmt_of(wl.F3)
    k, v = wl.prefill_kv(w, 0, 0)
    cache.append(0, [0], [1800], dev(k), dev(v))
    _sync()
    n = 1800 - w.window
    # oracle codes of other vectors, imported over the quantiser's
    rng = np.random.default_rng(3)
    ck, cv = [], []
    for kvh in range(w.n_kv_heads):
        xk = (rng.standard_normal((n, 128)) * 2).astype(np.float16)
        xv = rng.standard_normal((n, 128)).astype(np.float16)
        ck.append(codec.quantize(xk, pi, s, fm))
        cv.append(codec.quantize(xv, pi, s, fm))
        cache.import_codes(0, 0, kvh, 0, 0, codec.pack_records(ck[-1], 128, fm))
        cache.import_codes(0, 0, kvh, 1, 0, codec.pack_records(cv[-1], 128, fm))
        assert np.array_equal(cache.export_codes(0, 0, kvh, 1, 0, n), codec.pack_records(cv[-1], 128, fm))
    q = wl.query(w, 0, 0, 0)
    out = cache.attend(0, [0], dev(q[None])).cpu().numpy()[0]
    hk, hv = k[n:].transpose(1, 0, 2), v[n:].transpose(1, 0, 2)
    res = attention.decode_attention(q, hk, hv, ck, cv, np.ones(n, bool), pi, s, fm)
    assert_out_close(out, res["out"], "imported codes")


def test_value_qjl_off_tiny():
    """The tiny workload with polar-only values (v_qjl = 0): the value
    accumulation drops the sketch term, every output against the oracle's."""
    w = wl.make("tiny").with_(v_qjl=False)
    r = _run_paging(w, [0], w.steps)
    print("tiny v_qjl=0:", r)


def test_value_qjl_off_llama8b_slice_with_promotion():
    """Llama-3.1-8B-shaped heads, two sequences, polar-only values, promotion
    on (tau 0.15, sticky 3) with planted heavy hitters: outputs, and the
    promoted tokens' fp16 hot values (dequantised without the sketch term),
    against the oracle."""
    w = wl.make("llama8b").with_(n_seq=2, n_layers=1, prefill=(3000, 1337), formats=(wl.F3,), steps=12,
                                 tau=0.15, sticky=3, heavy_hitters=2, v_qjl=False)
    r = _run_paging(w, [0], w.steps)
    print("llama8b slice v_qjl=0:", r)
    assert r["promoted"] >= 2


def _gated_groups_from_logits(lg_row, cache, n_cold, g):
    """[H_kv] bool: groups whose cold debug logits are all -inf (not scored)."""
    cold = lg_row[:, cache.hot_capacity:cache.hot_capacity + n_cold]
    per_head = np.all(np.isneginf(cold), axis=1)
    return per_head.reshape(-1, g).all(axis=1)


def test_hot_first_gate_threshold_sweep():
    """Hot-first gated cold access ("Monarch v3", section "Bucle de
    Decodificacion Simplificado") on Llama-3.1-8B-shaped heads, two
    sequences: for thresholds from never-gated to always-gated, which kv
    groups skip their cold slots, the logits and the outputs, all against
    the oracle's gated step."""
    w = wl.make("llama8b").with_(n_seq=2, n_layers=1, prefill=(3000, 1337), formats=(wl.F3,), steps=1)
    seq_ids = [0, 1]
    cache = make_cache(w)
    fm = fmt_of(wl.F3)
    pi, s = oracle_params(w)
    oc = {sq: SeqLayerCache(w.n_kv_heads, w.head_dim, w.window, fm, pi, s) for sq in seq_ids}
    ks, vs = zip(*[wl.prefill_kv(w, 0, sq) for sq in seq_ids])
    cache.append(0, seq_ids, list(w.prefill), dev(np.concatenate(ks)), dev(np.concatenate(vs)))
    for i, sq in enumerate(seq_ids):
        oc[sq].append(ks[i], vs[i])
    _sync()
    for sq in seq_ids:
        _oracle_sync_codes(oc[sq], cache, sq, 0, f"prefill s{sq}")
    qs = [wl.query(w, 0, sq, 0) for sq in seq_ids]
    # each group's statistic (the smallest of its heads' best hot logits) is
    # its margin at threshold 0; thresholds between them gate some groups
    base = [oc[sq].attend(qs[i], gate=0.0)["gate_margin"] for i, sq in enumerate(seq_ids)]
    m = np.sort(np.concatenate(base))
    thetas = [float(m[len(m) // 4] + 1e-2), float(np.median(m) + 1e-2), float(m[-1] + 1.0), float(m[0] - 1.0)]
    g = w.n_q_heads // w.n_kv_heads
    n_gated = []
    for theta in thetas:
        import torch
        q = np.stack(qs)
        logits = torch.full((2, w.n_q_heads, cache.logits_stride), float("nan"), device="cuda")
        out = cache.attend(0, seq_ids, dev(q), logits=logits, gate=theta).cpu().numpy()
        _sync()
        logits = logits.cpu().numpy()
        tot = 0
        for i, sq in enumerate(seq_ids):
            res = oc[sq].attend(q[i], gate=theta)
            assert np.all(np.abs(res["gate_margin"]) > GATE_BAND)
            got = _gated_groups_from_logits(logits[i], cache, len(oc[sq].live), g)
            assert np.array_equal(got, res["gated"]), f"theta {theta} seq {sq}: {got} vs {res['gated']}"
            assert_out_close(out[i], res["out"], f"gated theta {theta} seq {sq}")
            nh = len(oc[sq].hot)
            assert_logits_close(logits[i, :, :nh], res["logits_hot"], f"gated theta {theta} seq {sq} hot")
            cold = logits[i, :, cache.hot_capacity:cache.hot_capacity + len(oc[sq].live)]
            assert_logits_close(cold, res["logits_cold"], f"gated theta {theta} seq {sq} cold")
            tot += int(res["gated"].sum())
        n_gated.append(tot)
        print(f"theta {theta:.3f}: {tot} of {2 * w.n_kv_heads} kv groups gated", flush=True)
    # a group gates when its statistic reaches the threshold: fewer at higher thresholds
    assert 2 * w.n_kv_heads > n_gated[0] > n_gated[1] > 0
    assert n_gated[2] == 0 and n_gated[3] == 2 * w.n_kv_heads


def test_hot_first_gate_with_promotion():
    """The gate inside the paging loop: gated steps record no cold candidates,
    so the sticky counters of their groups' hitters reset; TinyLlama-shaped
    heads with planted heavy hitters, 20 steps, hot FIFO, tombstones and
    counters against the oracle."""
    w = wl.make("tinyllama").with_(steps=20)
    r = _run_paging(w, [0], w.steps, gate=3.2)
    print("gated tinyllama:", r)
