"""Pins of the two oracle parts that only the decode path exercises (CPU).

1. The QJL term as the decode path computes it: the code-domain logit of
   attention.cold_logits and the QJL-inclusive dequantisation
   codec.dequantize.  "TurboQuant: kompresja KV-cache w LLM 6 razy"
   (sudonull.com, Polish), section "Kompensacja bledow przez QJL": the 1-bit
   Johnson-Lindenstrauss code of the residual keeps inner products unbiased.
   Over independent Gaussian sketches S the compressed logit is therefore an
   unbiased estimate of the exact one, <q, x> / sqrt(d) (Pi is orthogonal, so
   <Pi q, y_hat> + <Pi q, e> = <q, x>), up to the fp16 rounding of the stored
   residual norm; its spread has the closed form of the sign estimator:
   Var = [(pi/2) |q'|^2 |e|^2 - <q', e>^2] / m, times (rho / |e|)^2.  The
   dequantised vector's mean is x with total variance
   (pi/2) rho^2 (d - 2/pi) / m per sketch (each row s_j sign(s_j . e) has
   mean sqrt(2/pi) e/|e| and second moment d).

2. The boundary band (codec.boundary_band), checked against a brute-force
   geometric reading of "within tol of a decision boundary": the distance of
   the pair point to each decision half-line of the angle code (the rays
   half a bin off the grid angles), to each radius threshold circle
   (a + 1/2) R / (L_r - 1), and the distance of max r, |e| and every sketch
   projection z_j to the nearest fp16 rounding midpoint or to zero.
"""

import math

import numpy as np
import pytest

from oracle import attention, codec, params
from oracle.codec import Format

N_SEEDS = 10_000


def _aligned_query(pi, e, rng, d, align=0.6):
    """A query whose rotation q' = Pi q has a large component along e."""
    ehat = e / np.linalg.norm(e)
    qr = align * math.sqrt(d) * ehat + rng.standard_normal(d)
    return qr @ pi  # q = Pi^T q'


@pytest.mark.parametrize("fmt", [codec.F3, codec.F25])
def test_decode_path_qjl_term_unbiased_over_sketches(fmt):
    d = 128
    rng = np.random.default_rng(11)
    pi = params.rotation(d, 11)
    x16 = (rng.standard_normal((1, d)) * 1.7).astype(np.float16)
    x = x16.astype(np.float64)[0]
    # the polar part and the residual do not depend on the sketch
    c0 = codec.quantize(x16, pi, params.sketch(64, d, 0), fmt)
    e = c0["e"][0]
    ne = float(np.linalg.norm(e))
    assert abs(ne - 1.0) > 0.2  # so that rho and rho^2 differ
    q = _aligned_query(pi, e, rng, d)
    qr = pi @ q
    exact = float(q @ x) / math.sqrt(d)

    logit = np.empty(N_SEEDS)
    proj = np.empty(N_SEEDS)
    xsum = np.zeros(d)
    rho = None
    for k in range(N_SEEDS):
        s = params.sketch(64, d, 5000 + k)
        c = codec.quantize(x16, pi, s, fmt)
        logit[k] = attention.cold_logits(q[None], c, pi, s, fmt)[0, 0]
        xh = codec.dequantize(c, pi, s, fmt, qjl=True)[0]
        proj[k] = float(q @ xh) / math.sqrt(d)
        xsum += xh
        rho = float(c["rho16"][0])

    ratio = rho / ne
    var = ((math.pi / 2) * (qr @ qr) * ne ** 2 - float(qr @ e) ** 2) / fmt.m * ratio ** 2 / d
    sigma = math.sqrt(var)
    # the stored fp16 residual norm biases the estimate by (rho/|e| - 1) <q', e>
    rho_bias = abs(ratio - 1.0) * abs(float(qr @ e)) / math.sqrt(d)
    for name, est in (("cold_logits", logit), ("dequantize", proj)):
        assert abs(est.mean() - exact) <= 3.0 * sigma / math.sqrt(N_SEEDS) + rho_bias, name
        assert abs(est.std() / sigma - 1.0) < 0.03, name
    # the aligned component is large against the Monte Carlo band: a sign
    # flip, rho^2, a dropped sqrt(pi/2) or mismatched sketch rows move the
    # mean by at least a fifth of <q', e> / sqrt(d)
    assert 0.2 * abs(float(qr @ e)) / math.sqrt(d) > 10 * (3.0 * sigma / math.sqrt(N_SEEDS) + rho_bias)
    # vector mean of the dequantisation: E = x (up to rho's rounding) with
    # total variance (pi/2) rho^2 (d - 2/pi) / m per sketch
    mean = xsum / N_SEEDS
    want_bias = (ratio - 1.0) * (e @ pi)
    tv = (math.pi / 2) * rho ** 2 * (d - 2.0 / math.pi) / fmt.m / N_SEEDS
    r = float(np.sum((mean - x - want_bias) ** 2)) / tv
    assert 0.6 < r < 1.5, r


# ---------------------------------------------------------------- band pin

def _f16_midpoint_distance(v):
    """Distance of each v >= 0 to the nearest midpoint between consecutive
    fp16 values (brute force over the neighbours of fp16(v))."""
    v = np.asarray(v, dtype=np.float64)
    h = v.astype(np.float16)
    below = np.nextafter(h, np.float16(-np.inf)).astype(np.float64)
    above = np.nextafter(h, np.float16(np.inf)).astype(np.float64)
    hh = h.astype(np.float64)
    mids = np.stack([(below + hh) / 2.0, (hh + above) / 2.0])
    return np.abs(v[None] - mids).min(axis=0)


def _brute_band(c, s_full, fmt, band):
    y, e, z = c["y"], c["e"], c["z"]
    n, d = y.shape
    p = d // 2
    tol = band * np.linalg.norm(y, axis=1)
    R = c["R16"].astype(np.float64)
    lm1 = fmt.n_radius - 1
    pair = np.zeros((n, p), dtype=bool)
    L = fmt.n_angle
    rays = [(-np.pi + 2.0 * np.pi * (b + 0.5) / L) for b in range(L)]
    for i in range(n):
        for j in range(p):
            px, py = y[i, 2 * j], y[i, 2 * j + 1]
            r = math.hypot(px, py)
            near = False
            # decision half-lines of the angle code
            for psi in rays:
                ux, uy = math.cos(psi), math.sin(psi)
                along = px * ux + py * uy
                dist = abs(px * uy - py * ux) if along >= 0 else r
                near |= dist <= tol[i]
            # radius threshold circles
            if R[i] > 0:
                for a in range(lm1):
                    near |= abs(r - (a + 0.5) * R[i] / lm1) <= tol[i]
            pair[i, j] = near
    rmax = np.hypot(y[:, 0::2], y[:, 1::2]).max(axis=1)
    r_amb = _f16_midpoint_distance(rmax) <= tol
    pair |= r_amb[:, None]
    upstream = pair.any(axis=1) | r_amb
    rho = (_f16_midpoint_distance(np.linalg.norm(e, axis=1)) <= tol) | upstream
    snorm = np.linalg.norm(s_full[: fmt.m], axis=1)
    sign = (np.abs(z) <= tol[:, None] * snorm[None, :]) | upstream[:, None]
    vector = upstream | rho | sign.any(axis=1)
    return dict(pair=pair, R=r_amb, rho=rho, sign=sign, vector=vector)


@pytest.mark.parametrize("band", [1e-5, 1e-4])
@pytest.mark.parametrize("fmt", [codec.F3, codec.F4, codec.F25])
def test_boundary_band_equals_brute_force_geometry(fmt, band):
    d = 16
    rng = np.random.default_rng(21)
    pi = params.rotation(d, 21)
    s = params.sketch(64, d, 21)
    x = (rng.standard_normal((1500, d)) * rng.choice([0.02, 1.0, 40.0], size=(1500, 1))).astype(np.float16)
    c = codec.quantize(x, pi, s, fmt)
    got = codec.boundary_band(c, s, fmt, band=band)
    want = _brute_band(c, s, fmt, band)
    for k in ("pair", "R", "rho", "sign", "vector"):
        assert np.array_equal(got[k], want[k]), (k, int((got[k] != want[k]).sum()))
    # the sample must exercise every kind of flag without being all flagged
    assert 0 < want["pair"].sum() < want["pair"].size * 3 // 4
    assert 0 < want["R"].sum() < len(x) * 3 // 4
    indep = np.abs(c["z"]) <= band * np.linalg.norm(c["y"], axis=1)[:, None] * np.linalg.norm(s[: fmt.m], axis=1)
    assert indep.sum() > 0


def _pair_on(direction, radius, d=8):
    """A rotation that maps the first unit vector to the given pair direction
    in coordinates (0, 1), so that y = Pi e1 sits exactly there (fp64)."""
    u = np.zeros(d)
    u[0], u[1] = math.cos(direction), math.sin(direction)
    m = np.eye(d)
    m[:, 0] = u
    q, rr = np.linalg.qr(m)
    q = q * np.where(np.diag(rr) < 0, -1.0, 1.0)[None, :]
    assert np.allclose(q[:, 0], u)
    x = np.zeros((1, d), dtype=np.float16)
    x[0, 0] = radius
    return q, x


@pytest.mark.parametrize("fmt", [codec.F3, codec.F4, codec.F25])
def test_boundary_band_planted_rays_and_grid_angles(fmt):
    d = 8
    s = params.sketch(64, d, 2)
    L = fmt.n_angle
    for b in range(L):
        # exactly on a decision ray: flagged (the angle code is a tie)
        pi, x = _pair_on(-np.pi + 2 * np.pi * (b + 0.5) / L, 1.0, d)
        c = codec.quantize(x, pi, s, fmt)
        bb = codec.boundary_band(c, s, fmt)
        assert bb["pair"][0, 0] and bb["vector"][0], b
        # on a grid angle (the middle of a bin) at a radius that is the top
        # level: no flag on that pair
        pi, x = _pair_on(-np.pi + 2 * np.pi * b / L, 1.0, d)
        c = codec.quantize(x, pi, s, fmt)
        bb = codec.boundary_band(c, s, fmt)
        assert not bb["pair"][0, 0], b
        assert c["b"][0, 0] == b
