"""Seeded input generators: shapes, determinism and planted structure (CPU)."""

import numpy as np

from compressed_kv_decode_amd import workloads as wl


def test_shapes_and_determinism():
    w = wl.make("tiny")
    k, v = wl.prefill_kv(w, 0, 0)
    assert k.shape == (1024, 4, 64) and k.dtype == np.float16
    k2, _ = wl.prefill_kv(w, 0, 0)
    assert np.array_equal(k, k2)
    assert not np.array_equal(k, v)
    q = wl.query(w, 0, 0, 3)
    assert q.shape == (4, 64) and q.dtype == np.float16
    # 4 outlier channels x8 per kv head
    sc = wl.channel_scales(w, 0, "k")
    assert ((sc == 8.0).sum(axis=1) == 4).all()


def test_llama8b_outliers_one_percent():
    w = wl.make("llama8b")
    sc = wl.channel_scales(w, 3, "v")
    assert (sc == 10.0).sum() == 10 and sc.shape == (8, 128)


def test_ragged_lengths_range():
    w = wl.make("ragged")
    assert len(w.prefill) == 64
    assert min(w.prefill) >= 1024 and max(w.prefill) <= 16384
    assert 2000 < np.mean(w.prefill) < 9000
    assert w.formats[0] == wl.F3 and w.formats[1] == wl.F4


def test_heavy_hitter_schedule():
    w = wl.make("tinyllama")
    hh = wl.hitters(w, 5, 0)
    assert len(hh) == 2
    for tok, kv, on in hh:
        assert 0 <= tok < w.prefill[0] - w.window
        runs, cur = [], 1
        for a, b in zip(on, on[1:]):
            if b == a + 1:
                cur += 1
            else:
                runs.append(cur)
                cur = 1
        runs.append(cur)
        assert runs[:3] == [1, 2, 3]


def test_needle_geometry():
    w = wl.make("long").with_(prefill=(4096,))
    tok, u, kappa = wl.needle(w)
    k, _ = wl.prefill_kv(w, 0, 0, tok, tok + 1)
    q = wl.query(w, 0, 0, 0).astype(np.float64)
    # the needle key is kappa * u_g in every kv head; queries of group g point along u_g
    assert np.allclose(k[0].astype(np.float64), kappa * u, atol=1e-2)
    cos = (q[0] @ u[0]) / np.linalg.norm(q[0])
    assert cos > 0.95
