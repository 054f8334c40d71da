"""Pins of the compressed-vector MIPS oracle (CPU): the score is the
dequantised inner product, the selection is a brute-force sort, a fine code
converges to exact search, and recall rises with the bit width (the pages'
vector-search use of the codec: "Compresion del cache KV ... a 3 bits",
section "Aplicaciones mas alla de los LLMs")."""

import numpy as np
import pytest

from oracle import codec, mips, params
from oracle.codec import Format


def _db(n, d, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((n, d)).astype(np.float16), rng.standard_normal((6, d)).astype(np.float16)


def test_score_is_inner_product_with_dequantised_vector():
    d = 64
    x, q = _db(200, d, 1)
    pi, s = params.rotation(d, 1), params.sketch(64, d, 1)
    c = codec.quantize(x, pi, s, codec.F3)
    want = q.astype(np.float64) @ codec.dequantize(c, pi, s, codec.F3, qjl=True).T
    assert np.abs(mips.scores(q, c, pi, s, codec.F3) - want).max() < 1e-10


def test_topk_equals_brute_force_sort_with_ties_and_tombstones():
    rng = np.random.default_rng(2)
    sc = np.round(rng.standard_normal((5, 300)), 1)  # many exact ties
    live = rng.random(300) > 0.3
    idx, val = mips.topk(sc, 17, live)
    for r in range(5):
        cand = sorted(((-sc[r, j], j) for j in range(300) if live[j]))[:17]
        assert idx[r].tolist() == [j for _, j in cand]
        assert np.array_equal(val[r], np.array([-v for v, _ in cand]))
    idx2, val2 = mips.topk(sc[:, :4], 6)
    assert np.all(idx2[:, 4:] == -1) and np.all(np.isneginf(val2[:, 4:]))


def test_fine_codes_converge_to_exact_search():
    d = 64
    x, q = _db(2000, d, 3)
    pi, s = params.rotation(d, 3), params.sketch(64, d, 3)
    fine = Format(8, 10, 64)
    c = codec.quantize(x, pi, s, fine)
    got, _ = mips.topk(mips.scores(q, c, pi, s, fine), 10)
    truth, _ = mips.exact_topk(q, x, 10)
    assert mips.recall_at(got, truth) >= 0.95


@pytest.mark.parametrize("d", [64, 128])
def test_recall_rises_with_bit_width(d):
    x, q = _db(4000, d, 4)
    rng = np.random.default_rng(5)
    q = rng.standard_normal((40, d)).astype(np.float16)
    pi, s = params.rotation(d, 4), params.sketch(64, d, 4)
    truth, _ = mips.exact_topk(q, x, 10)
    rec = []
    for fmt in (codec.F25, codec.F3, codec.F4, Format(4, 6, 64)):
        c = codec.quantize(x, pi, s, fmt)
        got, _ = mips.topk(mips.scores(q, c, pi, s, fmt), 10)
        rec.append(mips.recall_at(got, truth))
    assert rec[0] < rec[1] < rec[2] < rec[3], rec
