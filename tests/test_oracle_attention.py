"""Pins of the oracle's decode attention (CPU)."""

import numpy as np
import pytest
import torch

from oracle import attention, codec, params
from oracle.codec import Format


@pytest.mark.parametrize("d", [4, 8, 64])
@pytest.mark.parametrize("fmt", [codec.F3, codec.F4, codec.F25])
def test_code_domain_logit_equals_dot_with_dequantised_key(d, fmt):
    rng = np.random.default_rng(d)
    pi, s = params.rotation(d, d), params.sketch(64, d, d)
    k = rng.standard_normal((32, d)).astype(np.float16)
    q = rng.standard_normal((3, d)).astype(np.float16)
    c = codec.quantize(k, pi, s, fmt)
    l_code = attention.cold_logits(q, c, pi, s, fmt)
    xh = codec.dequantize(c, pi, s, fmt, qjl=True)
    l_brute = q.astype(np.float64) @ xh.T / np.sqrt(d)
    assert np.abs(l_code - l_brute).max() < 1e-12


def test_hot_only_matches_torch_sdpa_cpu():
    rng = np.random.default_rng(1)
    hq, hkv, d, n = 8, 2, 64, 37
    q = rng.standard_normal((hq, d)).astype(np.float16)
    k = rng.standard_normal((hkv, n, d)).astype(np.float16)
    v = rng.standard_normal((hkv, n, d)).astype(np.float16)
    pi, s = params.rotation(d, 0), params.sketch(64, d, 0)
    res = attention.decode_attention(q, k, v, [None] * hkv, [None] * hkv, np.zeros(0, bool), pi, s, codec.F3)
    g = hq // hkv
    tq = torch.from_numpy(q.astype(np.float64)).view(hkv, g, 1, d)
    tk = torch.from_numpy(k.astype(np.float64)).view(hkv, 1, n, d).expand(hkv, g, n, d)
    tv = torch.from_numpy(v.astype(np.float64)).view(hkv, 1, n, d).expand(hkv, g, n, d)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv).reshape(hq, d).numpy()
    assert np.abs(res["out"] - ref).max() < 1e-12
    assert np.abs(attention.exact_attention(q, k, v) - ref).max() < 1e-12


def test_split_merge_equals_one_pass():
    rng = np.random.default_rng(2)
    logits = rng.standard_normal((4, 1000)) * 3
    vals = rng.standard_normal((1000, 16))
    full = attention.softmax(logits) @ vals
    cuts = [0, 1, 100, 101, 512, 999, 1000]
    states = [attention.partial_state(logits[:, a:b], vals[a:b]) for a, b in zip(cuts, cuts[1:])]
    assert np.abs(attention.merge_partials(states) - full).max() < 1e-12


def _mixed_cache(d=64, hkv=2, hq=4, n_hot=20, n_cold=50, fmt=codec.F3, seed=3):
    rng = np.random.default_rng(seed)
    pi, s = params.rotation(d, seed), params.sketch(64, d, seed)
    q = rng.standard_normal((hq, d)).astype(np.float16)
    hk = rng.standard_normal((hkv, n_hot, d)).astype(np.float16)
    hv = rng.standard_normal((hkv, n_hot, d)).astype(np.float16)
    ck = [codec.quantize(rng.standard_normal((n_cold, d)).astype(np.float16), pi, s, fmt) for _ in range(hkv)]
    cv = [codec.quantize(rng.standard_normal((n_cold, d)).astype(np.float16), pi, s, fmt) for _ in range(hkv)]
    live = rng.random(n_cold) > 0.2
    return q, hk, hv, ck, cv, live, pi, s


def test_permutation_invariance_and_tombstones():
    q, hk, hv, ck, cv, live, pi, s = _mixed_cache()
    base = attention.decode_attention(q, hk, hv, ck, cv, live, pi, s, codec.F3)
    perm = np.random.default_rng(9).permutation(len(live))
    keys = ("a", "b", "R16", "rho16", "signs")
    ckp = [{k: c[k][perm] for k in keys} for c in ck]
    cvp = [{k: c[k][perm] for k in keys} for c in cv]
    hp = np.random.default_rng(8).permutation(hk.shape[1])
    res = attention.decode_attention(q, hk[:, hp], hv[:, hp], ckp, cvp, live[perm], pi, s, codec.F3)
    assert np.abs(res["out"] - base["out"]).max() < 1e-12
    # a tombstoned slot has zero probability and its codes do not matter
    assert np.all(base["p_cold"][:, ~live] == 0.0)
    # probabilities sum to one over hot and live cold
    tot = base["p_hot"].sum(1) + base["p_cold"].sum(1)
    assert np.abs(tot - 1.0).max() < 1e-12


def test_fine_codes_converge_to_exact_attention():
    rng = np.random.default_rng(4)
    d, hkv, hq, n = 64, 2, 4, 200
    pi, s = params.rotation(d, 4), params.sketch(256, d, 4)
    q = rng.standard_normal((hq, d)).astype(np.float16)
    k = rng.standard_normal((hkv, n, d)).astype(np.float16)
    v = rng.standard_normal((hkv, n, d)).astype(np.float16)
    exact = attention.exact_attention(q, k, v)
    errs = []
    for fmt in (codec.F3, Format(4, 5, 64), Format(8, 8, 256)):
        ck = [codec.quantize(k[h], pi, s, fmt) for h in range(hkv)]
        cv = [codec.quantize(v[h], pi, s, fmt) for h in range(hkv)]
        empty = np.zeros((hkv, 0, d), np.float16)
        res = attention.decode_attention(q, empty, empty, ck, cv, np.ones(n, bool), pi, s, fmt, v_qjl=False)
        errs.append(np.abs(res["out"] - exact).max())
    assert errs[0] > errs[1] > errs[2]
    assert errs[2] < 1e-2


# ------------------------------------------------ hot-first gate ("Monarch v3",
# section "Bucle de Decodificacion Simplificado": cold pages are scored only
# when the best hot score is below a threshold)

def _sdpa_hot_only(q, hk, hv):
    """Textbook softmax attention over the hot tokens alone (torch, CPU, fp64)."""
    hq, d = q.shape
    hkv, n, _ = hk.shape
    g = hq // hkv
    tq = torch.from_numpy(q.astype(np.float64)).view(hkv, g, 1, d)
    tk = torch.from_numpy(hk.astype(np.float64)).view(hkv, 1, n, d).expand(hkv, g, n, d)
    tv = torch.from_numpy(hv.astype(np.float64)).view(hkv, 1, n, d).expand(hkv, g, n, d)
    return torch.nn.functional.scaled_dot_product_attention(tq, tk, tv).reshape(hq, d).numpy()


def test_gate_open_and_closed_special_cases():
    q, hk, hv, ck, cv, live, pi, s = _mixed_cache()
    base = attention.decode_attention(q, hk, hv, ck, cv, live, pi, s, codec.F3)
    opn = attention.decode_attention(q, hk, hv, ck, cv, live, pi, s, codec.F3, gate=np.inf)
    assert np.array_equal(opn["out"], base["out"]) and not opn["gated"].any()
    shut = attention.decode_attention(q, hk, hv, ck, cv, live, pi, s, codec.F3, gate=-np.inf)
    assert shut["gated"].all()
    assert np.abs(shut["out"] - _sdpa_hot_only(q, hk, hv)).max() < 1e-12
    assert np.all(shut["p_cold"] == 0.0) and np.all(np.isneginf(shut["logits_cold"]))


def test_gate_is_per_kv_group_and_any_head_below_opens_it():
    q, hk, hv, ck, cv, live, pi, s = _mixed_cache(hq=4, hkv=2)  # groups {0, 1}, {2, 3}
    d = q.shape[1]
    q = q.astype(np.float64)
    hk = hk.copy()
    # group 0: both heads find a hot key far above the threshold
    for h in (0, 1):
        hk[0, 3 + h] = (6.0 * q[h] / np.linalg.norm(q[h]) * np.sqrt(d) / np.linalg.norm(q[h]) * 2).astype(np.float16)
    # group 1: head 2 finds one, head 3 does not
    hk[1, 5] = (6.0 * q[2] / np.linalg.norm(q[2]) * np.sqrt(d) / np.linalg.norm(q[2]) * 2).astype(np.float16)
    q16 = q.astype(np.float16)
    theta = 8.0
    r = attention.decode_attention(q16, hk, hv, ck, cv, live, pi, s, codec.F3, gate=theta)
    lh = attention.hot_logits(q16, hk[0])
    assert lh[0].max() >= theta and lh[1].max() >= theta
    l1 = attention.hot_logits(q16[2:], hk[1])
    assert l1[0].max() >= theta and l1[1].max() < theta
    assert r["gated"].tolist() == [True, False]
    hot_only = _sdpa_hot_only(q16, hk, hv)
    assert np.abs(r["out"][:2] - hot_only[:2]).max() < 1e-12
    full = attention.decode_attention(q16, hk, hv, ck, cv, live, pi, s, codec.F3)
    assert np.abs(r["out"][2:] - full["out"][2:]).max() < 1e-12
    assert np.abs(r["out"][2:] - hot_only[2:]).max() > 1e-3  # the cold tokens matter there


def test_gate_closes_monotonically_with_the_threshold():
    q, hk, hv, ck, cv, live, pi, s = _mixed_cache(hq=8, hkv=4)
    prev = None
    for theta in np.linspace(4.0, -2.0, 25):
        g = attention.decode_attention(q, hk, hv, ck, cv, live, pi, s, codec.F3, gate=theta)["gated"]
        if prev is not None:
            assert np.all(g >= prev)  # a lower threshold gates at least the same groups
        prev = g
    assert prev.all()


# ------------------------------------------ multi-query (chunk / draft) attention

def test_multi_query_single_token_is_the_decode_step():
    q, hk, hv, ck, cv, live, pi, s = _mixed_cache()
    one = attention.multi_query_attention(q[None], hk, hv, ck, cv, live, pi, s, codec.F3, 1)
    base = attention.decode_attention(q, hk, hv, ck, cv, live, pi, s, codec.F3)
    assert np.array_equal(one[0], base["out"])


def test_multi_query_hot_only_equals_causal_sdpa():
    # no cold tokens: the chunk attends causally over the window, the older
    # entries visible to every query (torch SDPA with an explicit mask, CPU)
    rng = np.random.default_rng(7)
    hq, hkv, d, n_hot, n = 8, 2, 64, 30, 6
    q = rng.standard_normal((n, hq, d)).astype(np.float16)
    hk = rng.standard_normal((hkv, n_hot, d)).astype(np.float16)
    hv = rng.standard_normal((hkv, n_hot, d)).astype(np.float16)
    pi, s = params.rotation(d, 0), params.sketch(64, d, 0)
    got = attention.multi_query_attention(q, hk, hv, [None] * hkv, [None] * hkv, np.zeros(0, bool), pi, s, codec.F3, n)
    g = hq // hkv
    mask = np.ones((n, n_hot), dtype=bool)
    for j in range(n):
        mask[j, n_hot - n + j + 1:] = False
    for kv in range(hkv):
        tq = torch.from_numpy(q[:, kv * g:(kv + 1) * g].astype(np.float64)).permute(1, 0, 2)  # [g, n, d]
        tk = torch.from_numpy(hk[kv].astype(np.float64))[None].expand(g, n_hot, d)
        tv = torch.from_numpy(hv[kv].astype(np.float64))[None].expand(g, n_hot, d)
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(mask))
        assert np.abs(got[:, kv * g:(kv + 1) * g] - ref.permute(1, 0, 2).numpy()).max() < 1e-12


def test_multi_query_is_causal_within_the_chunk():
    q, hk, hv, ck, cv, live, pi, s = _mixed_cache(n_hot=20)
    rng = np.random.default_rng(8)
    n = 5
    qq = np.stack([q] * n) + rng.standard_normal((n,) + q.shape).astype(np.float16)
    a = attention.multi_query_attention(qq, hk, hv, ck, cv, live, pi, s, codec.F3, n)
    hk2, hv2 = hk.copy(), hv.copy()
    hk2[:, -2:] += 1.0  # change the chunk's last two tokens
    hv2[:, -2:] -= 2.0
    b = attention.multi_query_attention(qq, hk2, hv2, ck, cv, live, pi, s, codec.F3, n)
    assert np.array_equal(a[:n - 2], b[:n - 2])  # earlier queries never see them
    assert np.abs(a[n - 2:] - b[n - 2:]).max() > 1e-3
