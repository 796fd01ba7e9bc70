"""Lloyd-Max scalar codebook for the standard normal density (oracle side).

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.

Source: VeloxQuant "How I built" post, section "Stage 2: Lloyd-Max Scalar
Quantization" and "The Core Idea": the codebook is the fixed point of two
conditions, (1) every boundary is the midpoint of its two neighbouring
centroids and (2) every centroid is the conditional mean of the density over
its cell. The post iterates those two conditions from a starting guess; that is
what `lloyd_max` does first, in that order. Plain iteration slows to a crawl at
64+ levels, so the same fixed point is then polished with Newton steps on the
composed map (conditions (1) then (2)) minus the identity, using a
finite-difference Jacobian and numpy's dense solver. At 256 levels that map is
ill-conditioned (its Jacobian's smallest singular value is ~3e-5), so fp64
evaluation noise alone could move a centroid by ~1e-10; `lloyd_max_mp` therefore
evaluates the two conditions in mpmath at 40 digits and keeps correcting until
they hold to ~1e-30, far below fp32 resolution.

Readings (the pages leave these open):
  * 2^b levels for b bits (the PR's ratios need it; the post's 2^(b-1) is the
    residual variant).
  * Cell moments in closed form instead of the post's trapezoid quadrature:
    int_a^b x phi(x) dx = phi(a) - phi(b),  int_a^b phi = Q(a) - Q(b), with
    Q(x) = erfc(x / sqrt 2) / 2 evaluated on the tail side for accuracy.
  * Tables are rounded once to fp32 (round to nearest even) from the
    high-precision fixed point; each boundary is the exact midpoint of its two
    high-precision centroids, rounded once; the middle one is exactly 0.
"""
from __future__ import annotations

import functools
import math

import mpmath
import numpy as np
from scipy.special import erfc

_SQRT2 = math.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


def _phi(x):
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    fin = np.isfinite(x)
    out[fin] = _INV_SQRT_2PI * np.exp(-0.5 * x[fin] * x[fin])
    return out


def _upper_tail(x):
    """Q(x) = P(X > x) for X ~ N(0,1)."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * erfc(x / _SQRT2)


def _cell_mass(a, b):
    """P(a < X < b), evaluated on whichever side keeps the two terms small."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    out = np.empty_like(a)
    pos = a >= 0
    neg = b <= 0
    mid = ~(pos | neg)
    out[pos] = _upper_tail(a[pos]) - _upper_tail(b[pos])
    out[neg] = _upper_tail(-b[neg]) - _upper_tail(-a[neg])
    out[mid] = 1.0 - _upper_tail(-a[mid]) - _upper_tail(b[mid])
    return out


def _cell_first_moment(a, b):
    """int_a^b x phi(x) dx = phi(a) - phi(b) (phi(+-inf) = 0)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    pa, pb = _phi(a), _phi(b)
    out = pa - pb
    # phi(a) - phi(b) = phi(a) * (1 - exp(-(b^2 - a^2)/2)) keeps narrow cells exact
    fin = np.isfinite(a) & np.isfinite(b)
    out[fin] = -pa[fin] * np.expm1(-0.5 * (b[fin] - a[fin]) * (b[fin] + a[fin]))
    return out


def midpoints(c):
    """Condition (1): boundary k is the midpoint of centroids k and k+1."""
    c = np.asarray(c, dtype=np.float64)
    return 0.5 * (c[:-1] + c[1:])


def conditional_means(boundaries):
    """Condition (2): centroid of each cell (-inf, b0), (b0, b1), ..., (b_last, inf)."""
    b = np.asarray(boundaries, dtype=np.float64)
    lo = np.concatenate([[-np.inf], b])
    hi = np.concatenate([b, [np.inf]])
    return _cell_first_moment(lo, hi) / _cell_mass(lo, hi)


def lloyd_step(c):
    return conditional_means(midpoints(c))


def _symmetrise(c):
    c = np.asarray(c, dtype=np.float64)
    return 0.5 * (c - c[::-1])


@functools.lru_cache(maxsize=None)
def lloyd_max(bits: int, lloyd_iters: int = 2000, newton_iters: int = 30):
    """fp64 Lloyd-Max centroids for N(0,1) with 2^bits levels."""
    n = 1 << bits
    if n == 2:
        c = np.array([-1.0, 1.0])
    else:
        # spread the start over the bulk of the density
        c = np.linspace(-1.0, 1.0, n) * (1.0 + 0.9 * math.sqrt(2.0 * math.log(n)))
    # the pages' iteration: boundaries <- midpoints, centroids <- conditional means
    for _ in range(lloyd_iters):
        nxt = _symmetrise(lloyd_step(c))
        done = np.max(np.abs(nxt - c)) < 1e-15
        c = nxt
        if done:
            break
    # Newton polish of F(c) = lloyd_step(c) - c on the same fixed point
    for _ in range(newton_iters):
        f = lloyd_step(c) - c
        if np.max(np.abs(f)) < 1e-15:
            break
        jac = np.empty((n, n))
        for j in range(n):
            hstep = 1e-7 * max(1.0, abs(c[j]))
            e = np.zeros(n)
            e[j] = hstep
            jac[:, j] = ((lloyd_step(c + e) - (c + e)) - (lloyd_step(c - e) - (c - e))) / (2 * hstep)
        c = _symmetrise(c - np.linalg.solve(jac, f))
    return c


def residual(c):
    """Largest violation of the two conditions at centroids c (fp64)."""
    return float(np.max(np.abs(lloyd_step(c) - c)))


_MP_DPS = 40


def _lloyd_step_mp(c):
    """The composed map (midpoints, then conditional means) in mpmath at _MP_DPS digits."""
    n = len(c)
    b = [(c[i] + c[i + 1]) / 2 for i in range(n - 1)]
    out = []
    for i in range(n):
        lo = b[i - 1] if i > 0 else None
        hi = b[i] if i < n - 1 else None
        pa = mpmath.npdf(lo) if lo is not None else mpmath.mpf(0)
        pb = mpmath.npdf(hi) if hi is not None else mpmath.mpf(0)
        # P(lo < X < hi) through the upper tail on the side where it is small
        if lo is not None and lo >= 0:
            mass = mpmath.erfc(lo / mpmath.sqrt(2)) / 2 - (mpmath.erfc(hi / mpmath.sqrt(2)) / 2 if hi is not None else 0)
        elif hi is not None and hi <= 0:
            mass = mpmath.erfc(-hi / mpmath.sqrt(2)) / 2 - (mpmath.erfc(-lo / mpmath.sqrt(2)) / 2 if lo is not None else 0)
        else:
            ql = mpmath.erfc(-lo / mpmath.sqrt(2)) / 2 if lo is not None else mpmath.mpf(0)
            qh = mpmath.erfc(hi / mpmath.sqrt(2)) / 2 if hi is not None else mpmath.mpf(0)
            mass = 1 - ql - qh
        out.append((pa - pb) / mass)
    return out


@functools.lru_cache(maxsize=None)
def lloyd_max_mp(bits: int):
    """Centroids refined to ~1e-30: residual of the two conditions evaluated in
    mpmath, correction solved with the fp64 finite-difference Jacobian."""
    c64 = lloyd_max(bits)
    n = len(c64)
    jac = np.empty((n, n))
    for j in range(n):
        hstep = 1e-7 * max(1.0, abs(c64[j]))
        e = np.zeros(n)
        e[j] = hstep
        jac[:, j] = ((lloyd_step(c64 + e) - (c64 + e)) - (lloyd_step(c64 - e) - (c64 - e))) / (2 * hstep)
    with mpmath.workdps(_MP_DPS):
        c = [mpmath.mpf(float(x)) for x in c64]
        for _ in range(12):
            t = _lloyd_step_mp(c)
            f = [t[i] - c[i] for i in range(n)]
            if max(abs(x) for x in f) < mpmath.mpf(10) ** (-(_MP_DPS - 8)):
                break
            step = np.linalg.solve(jac, np.array([float(x) for x in f]))
            c = [c[i] - mpmath.mpf(float(step[i])) for i in range(n)]
            c = [(c[i] - c[n - 1 - i]) / 2 for i in range(n)]
        return tuple(c)


def residual_mp(bits: int) -> float:
    with mpmath.workdps(_MP_DPS):
        c = list(lloyd_max_mp(bits))
        t = _lloyd_step_mp(c)
        return float(max(abs(t[i] - c[i]) for i in range(len(c))))


def _round_f32(x) -> float:
    """Round an mpf to the nearest fp32 value (ties to even), returned as float."""
    man, exp = mpmath.frexp(x)           # x = man * 2**exp, 0.5 <= |man| < 1
    if man == 0:
        return 0.0
    scaled = man * mpmath.mpf(2) ** 24   # 24 significant bits
    r = mpmath.nint(scaled)              # mpmath nint rounds half to even
    return float(mpmath.ldexp(r, int(exp) - 24))


@functools.lru_cache(maxsize=None)
def tables(bits: int):
    """fp32 (centroids, boundaries) as the codec stores them: the high-precision
    fixed point rounded once to fp32; each boundary is the exact midpoint of its
    two high-precision centroids, rounded once."""
    c = lloyd_max_mp(bits)
    with mpmath.workdps(_MP_DPS):
        cent = np.array([_round_f32(x) for x in c], dtype=np.float32)
        bnd = np.array([_round_f32((c[i] + c[i + 1]) / 2) for i in range(len(c) - 1)],
                       dtype=np.float32)
    return cent, bnd


def distortion(c) -> float:
    """Mean squared error E[(X - Q(X))^2] of the codebook on N(0,1)."""
    c = np.asarray(c, dtype=np.float64)
    b = midpoints(c)
    lo = np.concatenate([[-np.inf], b])
    hi = np.concatenate([b, [np.inf]])
    mass = _cell_mass(lo, hi)
    m1 = _cell_first_moment(lo, hi)
    # int_a^b x^2 phi = mass + a phi(a) - b phi(b)
    fl, fh = np.isfinite(lo), np.isfinite(hi)
    apa = np.zeros_like(lo)
    bpb = np.zeros_like(hi)
    apa[fl] = lo[fl] * _phi(lo[fl])
    bpb[fh] = hi[fh] * _phi(hi[fh])
    m2 = mass + apa - bpb
    return float(np.sum(m2 - 2 * c * m1 + c * c * mass))
