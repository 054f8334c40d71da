"""Shared helpers of the GPU parity tests: build a library cache for a
workload, compare exported codes with the oracle's under the boundary band,
and compare attention results at the stated tolerances."""

import numpy as np

from compressed_kv_decode_amd import workloads as wl
from oracle import codec, params

LOGIT_RTOL = 1e-3   # |dl| <= 1e-3 * max(|l|, 1)
OUT_ATOL = 2e-3     # max-abs on fp32 outputs
# Vectors whose GPU record differs from the oracle's (each difference inside
# the boundary band, the oracle then adopts the GPU's choice).  The GPU's
# fp32 arithmetic is exact to about 2^-22 relative in the rotation and about
# 1e-7 relative in the pair radii and the residual norm, so a record differs
# only where a decision falls within that distance of its boundary: the fp16
# rounding of R or rho (about 2e-7 / 2^-11, a few 1e-4 per vector), a radius
# threshold, an angle ray or a sketch sign.  Measured: 1e-4 to 3.5e-4 on every
# workload; a kernel error that corrupted in-band vectors in bulk (about 1e-2
# of vectors sit in the band) would exceed the bound.
ADOPT_RATE = 1e-3
ADOPT_FLOOR = 3     # small samples: allow a few regardless of the rate


def assert_adoption(adopted, checked, what=""):
    """Adopted vectors are at most ADOPT_RATE of those checked (or the floor)."""
    rate = adopted / max(1, checked)
    print(f"adoption {what}: {adopted} of {checked} vectors ({rate:.2e})", flush=True)
    assert adopted <= max(ADOPT_FLOOR, ADOPT_RATE * checked), f"{what}: {adopted} of {checked} vectors adopted"
    return rate


def fmt_of(t):
    return codec.Format(*t)


def make_cache(w, n_seq_max=None, max_context=None, **over):
    from compressed_kv_decode_amd import tqkv
    kw = dict(n_seq_max=n_seq_max or w.n_seq, n_layers=w.n_layers, n_q_heads=w.n_q_heads,
              n_kv_heads=w.n_kv_heads, head_dim=w.head_dim, hot_window=w.window,
              max_context=max_context or w.max_context(), formats=list(w.formats), seed=w.seed,
              promote_threshold=w.tau, sticky=w.sticky, v_qjl=w.v_qjl)
    kw.update(over)
    return tqkv.Cache(**kw)


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def oracle_params(w, rotation_kind=0):
    """(Pi, S) of the oracle for a workload: the Haar rotation, or with
    rotation_kind 1 the randomized Hadamard one."""
    pi = params.hadamard_rotation(w.head_dim, w.seed) if rotation_kind else params.rotation(w.head_dim, w.seed)
    return pi, params.sketch(64, w.head_dim, w.seed)


def check_codes(gpu_rec, x16, pi, s_full, fmt, d, what=""):
    """Bit-exact outside the boundary band; inside it every differing field
    must be one the band marks.  Returns (oracle codes with the GPU's valid
    alternatives adopted, number of adopted vectors, number in the band)."""
    oc = codec.quantize(x16, pi, s_full, fmt)
    orec = codec.pack_records(oc, d, fmt)
    assert gpu_rec.shape == orec.shape, what
    diff = np.nonzero(np.any(gpu_rec != orec, axis=1))[0]
    band = codec.boundary_band(oc, s_full, fmt)
    if len(diff):
        g = codec.unpack_records(gpu_rec[diff], d, fmt)
        for n, i in enumerate(diff):
            pair_bad = (g["a"][n] != oc["a"][i]) | (g["b"][n] != oc["b"][i])
            assert not np.any(pair_bad & ~band["pair"][i]), f"{what}: vector {i} pair codes differ outside the band"
            assert g["R16"][n] == oc["R16"][i] or band["R"][i], f"{what}: vector {i} R differs"
            assert g["rho16"][n] == oc["rho16"][i] or band["rho"][i], f"{what}: vector {i} rho differs"
            sbad = g["signs"][n] != oc["signs"][i]
            assert not np.any(sbad & ~band["sign"][i]), f"{what}: vector {i} sign bits differ outside the band"
        adopted = dict(oc)
        for key in ("a", "b", "R16", "rho16", "signs"):
            adopted[key] = oc[key].copy()
            adopted[key][diff] = g[key]
        oc = adopted
    return oc, len(diff), int(band["vector"].sum())


def slice_codes(c, sl):
    return {k: c[k][sl] for k in ("a", "b", "R16", "rho16", "signs")}


def assert_logits_close(got, want, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    live = np.isfinite(want)
    assert np.array_equal(np.isfinite(got), live), f"{what}: live masks differ"
    err = np.abs(got[live] - want[live]) / np.maximum(np.abs(want[live]), 1.0)
    assert err.size == 0 or err.max() <= LOGIT_RTOL, f"{what}: logit rel err {err.max():.3e}"
    return float(err.max()) if err.size else 0.0


def assert_out_close(got, want, what=""):
    e = np.abs(np.asarray(got, dtype=np.float64) - want).max()
    assert e <= OUT_ATOL, f"{what}: output max-abs err {e:.3e}"
    return float(e)
