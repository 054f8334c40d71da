"""Error paths on the GPU, forced from the host with valid inputs: an fp16
radius scale that overflows (the kernels latch TQ_DEVERR_R_OVERFLOW and
clamp the scale, so every code stays in range), and a capacity overflow that
the host's mirror of appended tokens rejects before any launch.  "Monarch
v3" (openclawradar.com), section "Como funciona": evicted tokens are
quantised into the cold region; a vector whose largest rotated pair radius
does not fit the fp16 scale cannot be coded and is reported."""

import numpy as np
import pytest

from compressed_kv_decode_amd import tqkv
from compressed_kv_decode_amd import workloads as wl

from gpu_helpers import check_codes, dev, fmt_of, make_cache, oracle_params

pytestmark = pytest.mark.gpu

TQ_ERR_CAPACITY = 3
TQ_ERR_DEVICE = 6
TQ_DEVERR_R_OVERFLOW = 1


def _sync():
    import torch
    torch.cuda.synchronize()


@pytest.mark.parametrize("path", ["prefill", "decode_step"])
def test_radius_overflow_is_latched_and_other_sequences_are_coded(path):
    """Sequence 1 holds one vector with every component 60000: its rotated
    pair radii sum in square to |x|^2 = 128 * 60000^2, so the largest exceeds
    |x| / 8 = 85000 > 65504.  The error is latched; sequence 0's records
    (appended in the same calls) match the oracle."""
    d, W = 128, 64
    w = wl.make("llama8b").with_(n_seq=2, n_layers=1, prefill=(300, 300), formats=(wl.F3,), window=W, steps=0)
    cache = make_cache(w, max_context=400)
    pi, s = oracle_params(w)
    k0, v0 = wl.prefill_kv(w, 0, 0)
    k1, v1 = wl.prefill_kv(w, 0, 1)
    big = np.full((w.n_kv_heads, d), 60000.0, dtype=np.float16)
    # the overflowing vector is evicted by the prefill itself, or by the
    # decode-step append that pushes it out of the window
    at = 10 if path == "prefill" else w.prefill[1] - W
    k1 = k1.copy()
    k1[at] = big
    cache.append(0, [0, 1], [300, 300], dev(np.concatenate([k0, k1])), dev(np.concatenate([v0, v1])))
    xk0, xv0 = [k0], [v0]
    if path == "decode_step":
        for step in range(2):
            sk, sv = zip(*[wl.step_kv(w, 0, sq, step) for sq in (0, 1)])
            cache.append(0, [0, 1], [1, 1], dev(np.concatenate(sk)), dev(np.concatenate(sv)))
            xk0.append(sk[0])
            xv0.append(sv[0])
    _sync()
    st = cache.stats(0, 0)
    assert st["status"] == TQ_ERR_DEVICE, st
    assert st["device_error"] & TQ_DEVERR_R_OVERFLOW, st
    xk0, xv0 = np.concatenate(xk0), np.concatenate(xv0)
    nc = xk0.shape[0] - W
    assert st["cold_len"] == nc
    assert cache.stats(1, 0)["cold_len"] == nc
    fm = fmt_of(wl.F3)
    for kvh in range(w.n_kv_heads):
        check_codes(cache.export_codes(0, 0, kvh, 0, 0, nc), xk0[:nc, kvh], pi, s, fm, d, f"seq 0 kvh {kvh} K")
        check_codes(cache.export_codes(0, 0, kvh, 1, 0, nc), xv0[:nc, kvh], pi, s, fm, d, f"seq 0 kvh {kvh} V")
    # the overflowing vector's R is stored as the fp16 overflow (infinity)
    rec = cache.export_codes(1, 0, 0, 0, at, 1)
    r16 = rec[0, -4:-2].copy().view("<f2")[0]
    assert np.isinf(r16), r16


def test_capacity_is_checked_against_max_context_before_any_launch():
    w = wl.make("tiny").with_(prefill=(100,), steps=0)
    cache = make_cache(w, max_context=130)
    k, v = wl.prefill_kv(w, 0, 0)
    cache.append(0, [0], [100], dev(k), dev(v))
    # one token past max_context (which is not a multiple of the 32-slot tile)
    kk = np.concatenate([k, k])[:31]
    with pytest.raises(tqkv.TqError) as e:
        cache.append(0, [0], [31], dev(kk), dev(kk))
    assert e.value.status == TQ_ERR_CAPACITY
    _sync()
    st = cache.stats(0, 0)
    assert st["status"] == 0 and st["tokens_appended"] == 100 and st["hot_len"] == 100
    # exactly max_context is accepted
    cache.append(0, [0], [30], dev(kk[:30]), dev(kk[:30]))
    _sync()
    assert cache.stats(0, 0)["tokens_appended"] == 130
