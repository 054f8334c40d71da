"""Pins of the oracle codec: worked examples, brute force, bounds, byte
counts, bit-width monotonicity and the QJL estimator's statistics (CPU)."""

import json
import math
import os

import numpy as np
import pytest

from oracle import codec, params
from oracle.codec import Format

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_worked_examples_identity_rotation():
    g = json.load(open(os.path.join(GOLDEN, "codec_worked_examples.json")))
    for ex in g["examples"]:
        fmt = Format(*ex["format"])
        x = np.array([ex["x"]], dtype=np.float16)
        d = x.shape[1]
        s = np.array(ex["sketch_rows"], dtype=np.float64)
        c = codec.quantize(x, np.eye(d), s, fmt)
        assert c["a"][0].tolist() == ex["a"], ex["name"]
        assert c["b"][0].tolist() == ex["b"], ex["name"]
        assert float(c["R16"][0]) == ex["R16"]
        assert float(c["rho16"][0]) == ex["rho16"]
        assert c["signs"][0].astype(int).tolist() == ex["signs"]
        rec = codec.pack_records(c, d, fmt)
        assert rec[0].tobytes().hex() == ex["record_hex"], ex["name"]


@pytest.mark.parametrize("L", [4, 8, 16])
def test_angle_code_hand_values(L):
    fmt = Format(2, int(math.log2(L)), 32)
    # (1,0): angle 0 -> b = L/2; (0,1): pi/2 -> 3L/4; (-1,0): pi -> wraps to 0;
    # (0,-1): -pi/2 -> L/4; exact zero pair -> L/2
    y0 = np.array([[1.0, 0.0, -1.0, 0.0, 0.0]])
    y1 = np.array([[0.0, 1.0, 0.0, -1.0, 0.0]])
    b = codec.angle_code(y0, y1, fmt)[0].tolist()
    assert b == [L // 2, 3 * L // 4, 0, L // 4, L // 2]
    th = codec.angle_grid(fmt)
    assert th[L // 2] == 0.0 and abs(th[3 * L // 4] - np.pi / 2) < 1e-15 and th[0] == -np.pi


def _brute(r, theta, R, fmt):
    lv = np.arange(fmt.n_radius) * R / (fmt.n_radius - 1)
    a = int(np.argmin(np.abs(r - lv)))
    ph = codec.angle_grid(fmt)
    dist = np.abs(np.angle(np.exp(1j * (theta - ph))))
    b = int(np.argmin(dist))
    # distance gaps tell whether the brute-force winner is unambiguous
    ga = np.sort(np.abs(r - lv))
    gb = np.sort(dist)
    return a, b, ga[1] - ga[0], gb[1] - gb[0]


@pytest.mark.parametrize("fmt", [codec.F3, codec.F4, codec.F25, Format(1, 1, 32), Format(4, 4, 64)])
def test_brute_force_nearest_levels(fmt):
    rng = np.random.default_rng(2)
    d = 16
    x = (rng.standard_normal((300, d)) * rng.choice([0.01, 1.0, 30.0], size=(300, 1))).astype(np.float16)
    c = codec.quantize(x, np.eye(d), params.sketch(64, d, 0), fmt)
    xr = x.astype(np.float64)
    checked = 0
    for n in range(x.shape[0]):
        R = float(c["R16"][n])
        for i in range(d // 2):
            r = math.hypot(xr[n, 2 * i], xr[n, 2 * i + 1])
            th = math.atan2(xr[n, 2 * i + 1], xr[n, 2 * i])
            a, b, gapa, gapb = _brute(r, th, R, fmt)
            if gapa > 1e-9 * max(R, 1e-30):
                assert c["a"][n, i] == a
                checked += 1
            if r > 0 and gapb > 1e-9:
                assert c["b"][n, i] == b
    assert checked > 1000


@pytest.mark.parametrize("fmt", [codec.F3, codec.F4, codec.F25])
def test_per_pair_error_bounds(fmt):
    rng = np.random.default_rng(3)
    d = 64
    pi = params.rotation(d, 3)
    x = rng.standard_normal((500, d)).astype(np.float16)
    c = codec.quantize(x, pi, params.sketch(64, d, 3), fmt)
    R = c["R16"].astype(np.float64)[:, None]
    rhat = c["a"] * R / (fmt.n_radius - 1)
    ok = c["r"] <= R
    assert np.all(np.abs(c["r"] - rhat)[ok] <= R.repeat(d // 2, 1)[ok] / (2 * (fmt.n_radius - 1)) * (1 + 1e-12))
    # above R (R rounded down) the top level is used and the error is at most R's rounding
    assert np.all(c["a"][~ok] == fmt.n_radius - 1)
    th_hat = codec.angle_grid(fmt)[c["b"]]
    circ = np.abs(np.angle(np.exp(1j * (c["theta"] - th_hat))))
    assert np.all(circ <= np.pi / fmt.n_angle * (1 + 1e-12))


def test_record_bytes_closed_form():
    # B = ceil(P * (r_bits + theta_bits) / 8) + m / 8 + 4
    assert codec.record_bytes(64, codec.F3) == 28
    assert codec.record_bytes(128, codec.F3) == 48
    assert codec.record_bytes(64, codec.F4) == 40
    assert codec.record_bytes(128, codec.F4) == 68
    assert codec.record_bytes(64, codec.F25) == 28
    assert codec.record_bytes(128, codec.F25) == 44
    # the pair-code field of F3 at head_dim 64 is the 20 bytes per cold token
    # that the Monarch page quotes against 64-128 bytes hot
    assert codec.polar_bytes(64, codec.F3) == 20
    assert 2 * 64 == 128  # fp16 hot key at head_dim 64
    # nominal bits per value (codes + signs) at the defining head_dim
    assert (32 * 5 + 32) / 64 == 3.0
    assert (64 * 7 + 64) / 128 == 4.0
    assert (64 * 4 + 64) / 128 == 2.5
    # all-in ratio against fp16: F3 at head_dim 128 is 16/3
    assert abs(16.0 / codec.bits_per_value(128, codec.F3) - 16.0 / 3.0) < 1e-12


def test_pack_unpack_round_trip():
    rng = np.random.default_rng(4)
    for fmt, d in [(codec.F3, 64), (codec.F4, 128), (codec.F25, 128), (Format(3, 2, 32), 64)]:
        x = rng.standard_normal((50, d)).astype(np.float16)
        c = codec.quantize(x, params.rotation(d, 1), params.sketch(64, d, 1), fmt)
        rec = codec.pack_records(c, d, fmt)
        assert rec.shape == (50, codec.record_bytes(d, fmt))
        u = codec.unpack_records(rec, d, fmt)
        for k in ("a", "b", "signs", "R16", "rho16"):
            assert np.array_equal(u[k], c[k])


def _rel_mse(fmt, d, qjl, n=3000, seed=5):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, d)).astype(np.float16)
    pi, s = params.rotation(d, seed), params.sketch(64, d, seed)
    c = codec.quantize(x, pi, s, fmt)
    xh = codec.dequantize(c, pi, s, fmt, qjl=qjl)
    xx = x.astype(np.float64)
    return float(((xx - xh) ** 2).sum() / (xx ** 2).sum())


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("qjl", [False, True])
def test_reconstruction_error_falls_with_bits(d, qjl):
    chain = [codec.F25, codec.F3, codec.F4]
    errs = [_rel_mse(f, d, qjl) for f in chain]
    assert errs[0] > errs[1] > errs[2], errs
    # along the angle bits at fixed radius bits, and along radius bits at fixed angle bits
    e_t = [_rel_mse(Format(3, bt, 64), d, qjl) for bt in (2, 3, 4, 5)]
    assert all(a > b for a, b in zip(e_t, e_t[1:])), e_t
    e_r = [_rel_mse(Format(br, 4, 64), d, qjl) for br in (1, 2, 3, 4)]
    assert all(a > b for a, b in zip(e_r, e_r[1:])), e_r


def test_qjl_estimator_unbiased_and_closed_form_variance():
    d, m, n_seeds = 128, 64, 10_000
    rng = np.random.default_rng(6)
    q = rng.standard_normal(d)
    e = 0.3 * rng.standard_normal(d) + 0.2 * q
    est = np.empty(n_seeds)
    back = np.zeros(d)
    for k in range(n_seeds):
        s = params.sketch(m, d, 1000 + k)
        est[k] = codec.qjl_inner_product(q, e, s)
        back += s.T @ np.where(s @ e >= 0, 1.0, -1.0)
    true = float(q @ e)
    var_closed = (np.pi / 2 * (q @ q) * (e @ e) - true ** 2) / m
    sigma = math.sqrt(var_closed)
    assert abs(est.mean() - true) <= 3.0 * sigma / math.sqrt(n_seeds)
    assert abs(est.std() / sigma - 1.0) < 0.03
    # E[S^T sign(S e)] = m sqrt(2/pi) e / |e|
    back /= n_seeds
    want = m * math.sqrt(2.0 / np.pi) * e / np.linalg.norm(e)
    assert np.abs(back - want).max() < 4.0 * math.sqrt(m) / math.sqrt(n_seeds) * 1.5


def test_boundary_band_flags_planted_ties():
    # identity rotation: a pair placed exactly on a radius threshold and one on
    # an angle decision ray are inside the band; a generic vector is not.
    fmt = codec.F3
    d = 8
    s = params.sketch(64, d, 0)
    x = np.array([[3.0, 0.0, 1.5, 0.0, 0.7, 0.7, 0.1, -0.3],
                  [0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0],
                  [1.0, 0.3, -0.2, 0.9, 0.55, -0.6, 0.35, 0.25]], dtype=np.float16)
    c = codec.quantize(x, np.eye(d), s, fmt)
    bb = codec.boundary_band(c, s, fmt)
    # row 0: pair 1 has r = 1.5 = (1 + 1/2) * 3/3 -> on a radius threshold
    assert bb["pair"][0, 1]
    # row 1: all-zero vector: every angle code is at r = 0
    assert bb["pair"][1].all() and bb["vector"][1]
    assert not bb["vector"][2]
