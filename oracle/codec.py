"""PolarQuant pair codes plus the QJL 1-bit residual sketch (oracle, fp64).

Test infrastructure (see the package docstring).

Steps follow "TurboQuant: kompresja KV-cache w LLM 6 razy" (sudonull.com,
Polish), section "Zasada dzialania PolarQuant" (rotate at random, take radius
and angle, quantise them) and section "Kompensacja bledow przez QJL" (a 1-bit
code of the quantisation residual through a Johnson-Lindenstrauss
projection), in the order of the seven-step flow on "TurboQuant: optimizacion
de memoria para KV caches en inferencia de LLMs" (kerneldigest.dev): polar
mapping, polar quantisation, QJL correction, compressed store.

Readings taken where the pages are silent (each is one explicit choice):

* Pairs are adjacent coordinates (y[2i], y[2i+1]) of the rotated vector;
  radius r_i = hypot, angle theta_i = atan2(y[2i+1], y[2i]).
* Radius scale: R = fp16 round-to-nearest-even of max_i r_i, stored per
  vector; codes are binned against the stored R.
* Radius codebook: L_r = 2^r_bits levels a*R/(L_r-1), a = 0..L_r-1 (both
  ends representable); a = clamp(rint(r/R*(L_r-1)), 0, L_r-1) with
  round-half-even; R == 0 gives a = 0.
* Angle codebook: L_t = 2^theta_bits angles -pi + 2*pi*b/L_t;
  b = rint((theta+pi)*L_t/(2*pi)) mod L_t (nearest on the circle, pi wraps to
  -pi); an exactly zero pair takes b = L_t/2 (the code of angle 0).
* Residual e = y - y_hat; its norm is stored as fp16 (round-to-nearest-even).
* Sketch signs s_j = [ (S_m e)_j >= 0 ] for the first m rows of S (zero maps
  to bit 1); S acts on the rotated residual.
* Dequantisation x_hat = Pi^T (y_hat + sqrt(pi/2)/m * rho * S_m^T sigma) with
  sigma = 2s - 1 (the QJL term is the unbiased back-projection; switchable
  off for values).
* Canonical record (little-endian, least significant bit first): P codes
  c_i = a_i | (b_i << r_bits) at bit offset i*(r_bits+theta_bits), zero
  padded to a byte; then m sign bits; then R as fp16; then rho as fp16.
"""

from dataclasses import dataclass

import numpy as np

SQRT_HALF_PI = float(np.sqrt(np.pi / 2.0))


@dataclass(frozen=True)
class Format:
    """A code format: radius bits, angle bits, number of QJL sign bits."""

    r_bits: int
    theta_bits: int
    m: int

    @property
    def code_bits(self) -> int:
        return self.r_bits + self.theta_bits

    @property
    def n_radius(self) -> int:
        return 1 << self.r_bits

    @property
    def n_angle(self) -> int:
        return 1 << self.theta_bits


F3 = Format(2, 3, 32)
F4 = Format(3, 4, 64)
F25 = Format(2, 2, 64)


def polar_bytes(d: int, fmt: Format) -> int:
    """Bytes of the packed pair-code field of one vector."""
    return ((d // 2) * fmt.code_bits + 7) // 8


def record_bytes(d: int, fmt: Format) -> int:
    """Bytes of one canonical record: pair codes + sign bits + R + rho."""
    return polar_bytes(d, fmt) + (fmt.m + 7) // 8 + 4


def bits_per_value(d: int, fmt: Format) -> float:
    """All-in storage bits per original coordinate (codes + signs + scales)."""
    return record_bytes(d, fmt) * 8.0 / d


def to_f16(x) -> np.ndarray:
    """fp64 -> fp16 with round-to-nearest-even (numpy's direct conversion)."""
    return np.asarray(x, dtype=np.float64).astype(np.float16)


def angle_grid(fmt: Format) -> np.ndarray:
    return -np.pi + 2.0 * np.pi * np.arange(fmt.n_angle) / fmt.n_angle


def radius_code(r: np.ndarray, R: np.ndarray, fmt: Format) -> np.ndarray:
    """Nearest level of the closed radius grid {a*R/(L_r-1)} (stored R)."""
    lm1 = fmt.n_radius - 1
    R = np.asarray(R, dtype=np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(R > 0.0, r / np.where(R > 0.0, R, 1.0) * lm1, 0.0)
    return np.clip(np.rint(t), 0, lm1).astype(np.int64)


def angle_code(y0: np.ndarray, y1: np.ndarray, fmt: Format) -> np.ndarray:
    """Nearest grid angle on the circle; a zero pair takes the code of 0."""
    L = fmt.n_angle
    theta = np.arctan2(y1, y0)
    b = np.mod(np.rint((theta + np.pi) * L / (2.0 * np.pi)).astype(np.int64), L)
    zero = (y0 == 0.0) & (y1 == 0.0)
    return np.where(zero, L // 2, b)


def polar_reconstruct(a: np.ndarray, b: np.ndarray, R: np.ndarray, fmt: Format) -> np.ndarray:
    """y_hat (rotated domain) from pair codes and the stored radius scale."""
    rhat = a * (np.asarray(R, dtype=np.float64)[..., None] / (fmt.n_radius - 1))
    th = -np.pi + 2.0 * np.pi * b / fmt.n_angle
    out = np.empty(a.shape[:-1] + (2 * a.shape[-1],))
    out[..., 0::2] = rhat * np.cos(th)
    out[..., 1::2] = rhat * np.sin(th)
    return out


def quantize(x16: np.ndarray, pi: np.ndarray, s_full: np.ndarray, fmt: Format) -> dict:
    """Encode fp16 vectors x16 [N, d].

    Returns the codes (a, b, R16, rho16, signs) and the intermediate fp64
    values (y, r, theta, e, z) that the boundary-band analysis needs.
    """
    x = np.asarray(x16, dtype=np.float16).astype(np.float64)
    if x.ndim != 2:
        raise ValueError("x16 must be [N, d]")
    n, d = x.shape
    y = x @ pi.T
    y0, y1 = y[:, 0::2], y[:, 1::2]
    r = np.hypot(y0, y1)
    rmax = r.max(axis=1) if d > 0 else np.zeros(n)
    R16 = to_f16(rmax)
    if not np.all(np.isfinite(R16.astype(np.float64))):
        raise ValueError("radius scale overflows fp16")
    R = R16.astype(np.float64)
    a = radius_code(r, R, fmt)
    b = angle_code(y0, y1, fmt)
    yhat = polar_reconstruct(a, b, R, fmt)
    e = y - yhat
    rho16 = to_f16(np.linalg.norm(e, axis=1))
    sm = s_full[: fmt.m]
    z = e @ sm.T
    signs = z >= 0.0
    return dict(a=a, b=b, R16=R16, rho16=rho16, signs=signs,
                y=y, r=r, theta=np.arctan2(y1, y0), e=e, z=z, yhat=yhat)


def pack_records(codes: dict, d: int, fmt: Format) -> np.ndarray:
    """Canonical byte records [N, record_bytes]."""
    a, b = codes["a"], codes["b"]
    n, p = a.shape
    cb = fmt.code_bits
    c = (a | (b << fmt.r_bits)).astype(np.uint64)
    shifts = np.arange(cb, dtype=np.uint64)
    bits = ((c[:, :, None] >> shifts[None, None, :]) & np.uint64(1)).astype(np.uint8)
    bits = bits.reshape(n, p * cb)
    pb = polar_bytes(d, fmt)
    polar = np.zeros((n, pb * 8), dtype=np.uint8)
    polar[:, : p * cb] = bits
    polar = np.packbits(polar, axis=1, bitorder="little")
    sb = (fmt.m + 7) // 8
    sbits = np.zeros((n, sb * 8), dtype=np.uint8)
    sbits[:, : fmt.m] = codes["signs"].astype(np.uint8)
    sgn = np.packbits(sbits, axis=1, bitorder="little")
    r16 = codes["R16"].astype("<f2").view(np.uint8).reshape(n, 2)
    rho = codes["rho16"].astype("<f2").view(np.uint8).reshape(n, 2)
    return np.concatenate([polar, sgn, r16, rho], axis=1)


def unpack_records(rec: np.ndarray, d: int, fmt: Format) -> dict:
    """Inverse of pack_records."""
    rec = np.asarray(rec, dtype=np.uint8)
    n = rec.shape[0]
    p = d // 2
    cb = fmt.code_bits
    pb = polar_bytes(d, fmt)
    sb = (fmt.m + 7) // 8
    bits = np.unpackbits(rec[:, :pb], axis=1, bitorder="little")[:, : p * cb]
    bits = bits.reshape(n, p, cb).astype(np.int64)
    c = (bits << np.arange(cb)[None, None, :]).sum(axis=2)
    a = c & ((1 << fmt.r_bits) - 1)
    b = c >> fmt.r_bits
    signs = np.unpackbits(rec[:, pb: pb + sb], axis=1, bitorder="little")[:, : fmt.m].astype(bool)
    R16 = rec[:, pb + sb: pb + sb + 2].copy().view("<f2").reshape(n).astype(np.float16)
    rho16 = rec[:, pb + sb + 2: pb + sb + 4].copy().view("<f2").reshape(n).astype(np.float16)
    return dict(a=a, b=b, R16=R16, rho16=rho16, signs=signs)


def qjl_backprojection(codes: dict, s_full: np.ndarray, fmt: Format) -> np.ndarray:
    """sqrt(pi/2)/m * rho * S_m^T sigma in the rotated domain, [N, d]."""
    sigma = 2.0 * codes["signs"].astype(np.float64) - 1.0
    rho = codes["rho16"].astype(np.float64)
    return (SQRT_HALF_PI / fmt.m) * rho[:, None] * (sigma @ s_full[: fmt.m])


def dequantize_rotated(codes: dict, s_full: np.ndarray, fmt: Format, qjl: bool = True) -> np.ndarray:
    """Reconstruction in the rotated domain: y_hat (+ QJL back-projection)."""
    yh = polar_reconstruct(codes["a"], codes["b"], codes["R16"].astype(np.float64), fmt)
    if qjl:
        yh = yh + qjl_backprojection(codes, s_full, fmt)
    return yh


def dequantize(codes: dict, pi: np.ndarray, s_full: np.ndarray, fmt: Format, qjl: bool = True) -> np.ndarray:
    """x_hat = Pi^T (y_hat + QJL term), original domain, [N, d] fp64."""
    return dequantize_rotated(codes, s_full, fmt, qjl) @ pi


def qjl_inner_product(q: np.ndarray, e: np.ndarray, s_m: np.ndarray) -> float:
    """QJL estimate of <q, e>: sqrt(pi/2)/m * ||e|| * <S q, sign(S e)>."""
    m = s_m.shape[0]
    sg = np.where(s_m @ e >= 0.0, 1.0, -1.0)
    return SQRT_HALF_PI / m * np.linalg.norm(e) * float((s_m @ q) @ sg)


def f16_rounding_ambiguous(v: np.ndarray, tol: np.ndarray) -> np.ndarray:
    """True where fp16 rounding of v could change within +-tol."""
    v = np.asarray(v, dtype=np.float64)
    return to_f16(v - tol) != to_f16(v + tol)


def boundary_band(codes: dict, s_full: np.ndarray, fmt: Format, band: float = 1e-6) -> dict:
    """Which fields sit within band*||y|| of a decision boundary.

    A GPU computing in fp32 may legitimately decide these the other way.
    Returns boolean masks: 'pair' [N, P] (radius or angle code near a bin
    edge), 'R' [N], 'rho' [N], 'sign' [N, m], and 'vector' [N] (any of them).
    An ambiguous R or pair code makes that vector's rho and signs ambiguous
    too (they are computed from the reconstruction).
    """
    y, r, theta, e, z = codes["y"], codes["r"], codes["theta"], codes["e"], codes["z"]
    ny = np.linalg.norm(y, axis=1)
    tol = band * ny
    R = codes["R16"].astype(np.float64)
    lm1 = fmt.n_radius - 1
    # radius: distance to the nearest half-level threshold (a+1/2)*R/(L_r-1)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(R[:, None] > 0, r * lm1 / np.where(R[:, None] > 0, R[:, None], 1.0), 0.0)
    half = np.clip(np.rint(t - 0.5), 0, lm1 - 1) + 0.5
    drad = np.abs(t - half) * (R[:, None] / lm1)
    rad_amb = (R[:, None] > 0) & (drad <= tol[:, None])
    # angle: distance from the pair to the nearest decision ray (rays within a
    # quarter turn only: sin also vanishes on the opposite ray)
    L = fmt.n_angle
    rays = -np.pi + 2.0 * np.pi * (np.arange(L) + 0.5) / L
    diff = theta[:, :, None] - rays[None, None, :]
    dist = np.where(np.cos(diff) > 0, np.abs(r[:, :, None] * np.sin(diff)), np.inf).min(axis=2)
    ang_amb = (dist <= tol[:, None]) | (r <= tol[:, None])
    pair = rad_amb | ang_amb
    rmax = r.max(axis=1)
    R_amb = f16_rounding_ambiguous(rmax, tol)
    pair = pair | R_amb[:, None]
    rho_amb = f16_rounding_ambiguous(np.linalg.norm(e, axis=1), tol)
    snorm = np.linalg.norm(s_full[: fmt.m], axis=1)
    sign = np.abs(z) <= tol[:, None] * snorm[None, :]
    upstream = pair.any(axis=1) | R_amb
    rho_amb = rho_amb | upstream
    sign = sign | upstream[:, None]
    vector = upstream | rho_amb | sign.any(axis=1)
    return dict(pair=pair, R=R_amb, rho=rho_amb, sign=sign, vector=vector)
