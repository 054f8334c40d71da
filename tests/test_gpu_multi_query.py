"""Multi-query attention over the compressed cache on the GPU against the
oracle: the queries of the newest n tokens of a sequence (a prefill chunk
or draft tokens), causal within the chunk, over cold codes and the hot
window.  Group sizes and chunk lengths cover one pass of 8 virtual heads,
padded passes and several passes."""

import numpy as np
import pytest

from compressed_kv_decode_amd import workloads as wl
from oracle import attention
from oracle.paging import SeqLayerCache

from gpu_helpers import assert_out_close, dev, fmt_of, make_cache, oracle_params
from test_gpu_parity import _oracle_sync_codes

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("hq,hkv,d,fmt,prefill,n", [
    (32, 8, 128, wl.F3, 3000, 5),    # G 4: 20 virtual heads per kv head, passes 8 + 8 + 4
    (4, 4, 64, wl.F4, 1500, 8),      # G 1: one pass of 8
    (8, 1, 128, wl.F25, 2100, 3),    # G 8: three passes
    (8, 4, 64, wl.F3, 700, 3),       # G 2: 6 virtual heads, one padded pass of 8
    (32, 8, 128, wl.F3, 300, 4),     # no cold tokens (context within the window)
])
def test_multi_query_against_oracle(hq, hkv, d, fmt, prefill, n):
    import torch
    w = wl.make("llama8b").with_(n_seq=2, n_layers=1, n_q_heads=hq, n_kv_heads=hkv, head_dim=d, formats=(fmt,),
                                 prefill=(prefill, 999), steps=n, window=512)
    cache = make_cache(w, n_seq_max=2, max_context=prefill + n + 8)
    pi, s = oracle_params(w)
    oc = SeqLayerCache(hkv, d, w.window, fmt_of(fmt), pi, s)
    k, v = wl.prefill_kv(w, 0, 0)
    cache.append(0, [0], [prefill], dev(k), dev(v))
    oc.append(k, v)
    # the chunk: n new tokens in one append
    rng = np.random.default_rng(prefill + n)
    ck = rng.standard_normal((n, hkv, d)).astype(np.float16)
    cv = rng.standard_normal((n, hkv, d)).astype(np.float16)
    cache.append(0, [0], [n], dev(ck), dev(cv))
    oc.append(ck, cv)
    torch.cuda.synchronize()
    _oracle_sync_codes(oc, cache, 0, 0, "multi-query store")
    q = rng.standard_normal((n, hq, d)).astype(np.float16)
    # a workspace full of NaN: nothing the call does not write may reach the output
    import ctypes
    nb = ctypes.c_size_t(0)
    cache.lib.tq_multi_query_workspace_bytes(cache.h, ctypes.byref(nb))
    ws = torch.full((nb.value // 4 + 64,), float("nan"), device="cuda").view(torch.uint8)
    out = cache.multi_query(0, 0, dev(q), workspace=ws).cpu().numpy()
    hk, hv = oc.hot_arrays()
    cks = [oc.cold_codes(kv, "k") for kv in range(hkv)]
    cvs = [oc.cold_codes(kv, "v") for kv in range(hkv)]
    want = attention.multi_query_attention(q, hk, hv, cks, cvs, np.array(oc.live, bool), pi, s, fmt_of(fmt), n)
    for j in range(n):
        assert_out_close(out[j], want[j], f"G {hq // hkv} n {n} token {j}")
    # the call is no decode step: the layer's attention counter is unchanged
    st = cache.stats(0, 0)
    assert st["status"] == 0 and st["attn_steps"] == 0
    # its last query is the decode step of the newest token
    last = cache.attend(0, [0], dev(q[-1:])).cpu().numpy()[0]
    assert np.abs(last - out[-1]).max() <= 2e-3


# The G 2 case at head_dim 64 (one outlier channel of ten times the scale in
# 64, so large value pair radii) measured 2.08e-3 against the oracle, over the
# 2e-3 bar, while the value tables held the unit values rounded to fp16 as
# they are (an output moves by up to max R / 4096 that way).  The tables now
# hold them times a per-format scale under which they round to fp16 within
# about 1e-16 (F2.5), 1e-6 (F3) and 7e-5 (F4) of their size.
BATCH_CASES = [
    pytest.param(32, 8, 128, wl.F3, (3000, 1337, 300), 3, id="G4-d128-F3"),  # 12 virtual heads, passes 8 + 4; third sequence all hot
    pytest.param(8, 1, 128, wl.F4, (2100, 900), 2, id="G8-d128-F4"),         # two passes
    pytest.param(8, 4, 64, wl.F25, (700, 1500, 1100, 64), 5, id="G2-d64-F25"),  # 10 virtual heads, passes 8 + 2
]


def _batch_case(hq, hkv, d, fmt, prefill, n):
    """Several sequences, each with its own context length and its newest n
    tokens as the chunk, in one tq_multi_query_attention_batch call (in a
    shuffled sequence order, NaN-filled workspace); returns per sequence
    (batch output, one-sequence call output, oracle output)."""
    import torch
    n_seq = len(prefill)
    w = wl.make("llama8b").with_(n_seq=n_seq, n_layers=1, n_q_heads=hq, n_kv_heads=hkv, head_dim=d,
                                 formats=(fmt,), prefill=prefill, steps=n, window=512)
    cache = make_cache(w, n_seq_max=n_seq, max_context=max(prefill) + n + 8)
    pi, s = oracle_params(w)
    rng = np.random.default_rng(sum(prefill) + n)
    seqs = list(range(n_seq))
    oc, qs = [], []
    for sq in seqs:
        o = SeqLayerCache(hkv, d, w.window, fmt_of(fmt), pi, s)
        k, v = wl.prefill_kv(w, 0, sq)
        cache.append(0, [sq], [prefill[sq]], dev(k), dev(v))
        o.append(k, v)
        ck = rng.standard_normal((n, hkv, d)).astype(np.float16)
        cv = rng.standard_normal((n, hkv, d)).astype(np.float16)
        cache.append(0, [sq], [n], dev(ck), dev(cv))
        o.append(ck, cv)
        oc.append(o)
        qs.append(rng.standard_normal((n, hq, d)).astype(np.float16))
    torch.cuda.synchronize()
    for sq in seqs:
        _oracle_sync_codes(oc[sq], cache, sq, 0, f"multi-query batch store seq {sq}")
    order = seqs[::-1]
    q = np.stack([qs[sq] for sq in order])
    nb = cache.multi_query_batch_workspace_bytes(n_seq)
    ws = torch.full((nb // 4 + 64,), float("nan"), device="cuda").view(torch.uint8)
    out = cache.multi_query_batch(0, order, dev(q), workspace=ws).cpu().numpy()
    res = {}
    for i, sq in enumerate(order):
        o = oc[sq]
        hk, hv = o.hot_arrays()
        cks = [o.cold_codes(kv, "k") for kv in range(hkv)]
        cvs = [o.cold_codes(kv, "v") for kv in range(hkv)]
        want = attention.multi_query_attention(qs[sq], hk, hv, cks, cvs, np.array(o.live, bool), pi, s,
                                               fmt_of(fmt), n)
        one = cache.multi_query(0, sq, dev(qs[sq])).cpu().numpy()
        print(f"seq {sq}: batch vs one-sequence call {np.abs(out[i] - one).max():.2e}, batch vs oracle "
              f"{np.abs(out[i] - want).max():.2e}", flush=True)
        res[sq] = (out[i], one, want)
    st = cache.stats(0, 0)
    assert st["status"] == 0 and st["attn_steps"] == 0
    return res


@pytest.mark.parametrize("hq,hkv,d,fmt,prefill,n", BATCH_CASES)
def test_multi_query_batch_equals_one_sequence_calls(hq, hkv, d, fmt, prefill, n):
    """The batch call computes what the one-sequence calls compute: the
    same kernels over the same codes, only the split of each stream into
    parts (and so the order of the merge) differs."""
    for sq, (out, one, _) in _batch_case(hq, hkv, d, fmt, prefill, n).items():
        assert np.abs(out - one).max() <= 1e-4, f"seq {sq}: batch against one-sequence call"


@pytest.mark.parametrize("hq,hkv,d,fmt,prefill,n", BATCH_CASES)
def test_multi_query_batch_against_oracle(hq, hkv, d, fmt, prefill, n):
    """Every sequence's outputs of the batch call against the oracle."""
    for sq, (out, _, want) in _batch_case(hq, hkv, d, fmt, prefill, n).items():
        for j in range(n):
            assert_out_close(out[j], want[j], f"batch G {hq // hkv} seq {sq} token {j}")
