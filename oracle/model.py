"""Probability model, integer rANS table, rate table and lambda grid.

Follows [D-Quant] §3.1 (rANS with precision p, integer frequencies f_m summing
to 2^p, a 2^p-entry decode table), §4.2 (the entropy model is derived from
Gaussian order statistics; affine invariance lets one table serve every token
and layer), §4.4 "Distribution sharpening" (p'_m proportional to p_m^alpha) and
Appendix A, Algorithm 1 (r_m = -log2(f_m / sum f)).

Readings (the page does not spell these out):
  * The model p_m(M, n) is the expected fraction of level m when n iid N(0,1)
    values are min-max normalised (Eq. 4) and rounded to the nearest of the M
    levels.  Appendix A lets a table entry carry any reconstruction level v_m;
    with non-affine levels (v_0 = 0 < ... < v_{M-1} = M - 1 in grid units) the
    cells of nearest rounding are bounded by the midpoints of adjacent levels,
    and the model is symmetrised only when the levels are symmetric.  The minimum always lands on level 0 and the maximum on level M-1;
    the other n-2 values are iid N(0,1) truncated to (min, max).  It is
    evaluated by 2-D Gauss-Legendre quadrature in float64 and symmetrised
    (p_m and p_{M-1-m} are equal by symmetry of the normal law; averaging them
    makes that exact so that tie-breaks below are reproducible).
  * Integer table: f_m = max(1, floor(256 q_m)); missing units go one each to
    the largest remainders 256 q_m - f_m (ties to the lower index); any excess
    is taken one unit at a time from the largest f (ties to the lower index).
  * Rates are fixed point: r_fx[m] = rne((8 - log2 f_m) * 2^16), so the rate
    of a stream is an exact integer sum; the container budget is
    B_fx = (8C - 32) * 2^16 (Eq. 3 with a 32-bit final state).
  * Lambda grid: E[k] = fp32(2^(k/512)) correctly rounded, k = 0..511, so that
    2^u for u on a 1/512 grid is ldexp(E[u mod 512], floor(u / 512)).
"""

import numpy as np
from scipy import special

PROB_BITS = 8                 # p: low 8 state bits index a 256-entry table
SIGMA_BITS = 32               # final-state overhead: one 32-bit state
L_RANS = 1 << 23              # lower end of the normalised state interval
RATE_FRAC_BITS = 16


def level_midpoints(M, values=None):
    """Cell boundaries, in grid units, of nearest rounding to the M levels:
    (v_{m-1} + v_m) / 2 for m = 1..M-1 (affine levels v_m = m give m - 1/2)."""
    if values is None:
        return np.arange(1, M, dtype=np.float64) - 0.5
    v = np.asarray(values, np.float64)
    return 0.5 * (v[:-1] + v[1:])


def levels_symmetric(M, values=None):
    """True if v_m + v_{M-1-m} == M - 1 exactly for every m."""
    if values is None:
        return True
    v = np.asarray(values, np.float64)
    return bool(np.all(v + v[::-1] == float(M - 1)))


def order_stat_probs(M, n, nodes=512, lo=-9.0, hi=9.0, values=None):
    """p_m(M, n) in float64 (see module docstring), symmetrised when the
    levels are.  ``values`` are non-affine level positions in grid units
    (v_0 = 0, v_{M-1} = M - 1, increasing); None means v_m = m."""
    if M < 2 or n < 2:
        raise ValueError("need M >= 2 and n >= 2")
    mids = level_midpoints(M, values)
    p = np.zeros(M, np.float64)
    p[0] += 1.0
    p[M - 1] += 1.0
    if n > 2:
        t, w = np.polynomial.legendre.leggauss(nodes)
        a = 0.5 * (hi - lo) * t + 0.5 * (hi + lo)          # outer: the minimum
        wa = 0.5 * (hi - lo) * w
        half = 0.5 * (hi - a)
        b = half[:, None] * t[None, :] + (0.5 * (hi + a))[:, None]   # inner: max in (a, hi)
        wb = half[:, None] * w[None, :]
        A = np.broadcast_to(a[:, None], b.shape)
        # Phi(b) - Phi(a) without cancellation in the bulk of the mass
        G = 1.0 - special.ndtr(A) - special.ndtr(-b)
        G = np.maximum(G, 0.0)
        phi = lambda v: np.exp(-0.5 * v * v) / np.sqrt(2.0 * np.pi)
        # joint density of (min, max) times 1/(Phi(b)-Phi(a)) for the
        # truncated law of an interior value
        dens = float(n) * float(n - 1) * phi(A) * phi(b) * np.power(G, n - 3)
        wts = wa[:, None] * wb * dens
        width = b - A
        for m in range(M):
            lo_u = mids[m - 1] if m > 0 else -0.5
            hi_u = mids[m] if m < M - 1 else M - 0.5
            e_lo = np.clip(A + width * (lo_u / (M - 1)), A, b)
            e_hi = np.clip(A + width * (hi_u / (M - 1)), A, b)
            cell = special.ndtr(e_hi) - special.ndtr(e_lo)
            p[m] += float(n - 2) * float(np.sum(wts * cell))
    p /= float(n)
    if not levels_symmetric(M, values):
        return p
    sym = np.empty_like(p)
    for m in range(M):
        sym[m] = (p[m] + p[M - 1 - m]) / 2.0
    return sym


def level_values_fp16(M, values=None):
    """The reconstruction levels as stored in the table: float16, returned as
    float32 (v_m = m when values is None).  Raises unless v_0 = 0,
    v_{M-1} = M - 1 and the levels strictly increase after rounding."""
    if values is None:
        return np.arange(M, dtype=np.float32)
    v = np.asarray(values, np.float64)
    if v.shape != (M,):
        raise ValueError("need one value per level")
    v16 = v.astype(np.float32).astype(np.float16).astype(np.float32)
    if v16[0] != 0.0 or v16[-1] != float(M - 1) or not np.all(np.diff(v16) > 0):
        raise ValueError("levels must rise strictly from 0 to M - 1")
    return v16


def sharpen(p, alpha):
    """q_m = p_m^alpha / sum_j p_j^alpha (§4.4), sum taken in index order."""
    pa = np.power(np.asarray(p, np.float64), float(alpha))
    tot = 0.0
    for v in pa:
        tot += float(v)
    return pa / tot


def integer_table(q, total=1 << PROB_BITS):
    """Integer frequencies f (sum = 256, every f >= 1) from probabilities q."""
    q = np.asarray(q, np.float64)
    M = len(q)
    raw = q * float(total)
    f = np.maximum(1, np.floor(raw)).astype(np.int64)
    missing = total - int(f.sum())
    if missing > 0:
        rem = raw - f
        order = sorted(range(M), key=lambda m: (-rem[m], m))
        for m in order[:missing]:
            f[m] += 1
    while int(f.sum()) > total:
        m = int(np.argmax(f))          # first index of the largest count
        f[m] -= 1
    if int(f.sum()) != total or f.min() < 1:
        raise ValueError("could not build an integer table")
    return f


def build_table(M, n, alpha, values=None):
    """(f, c): frequencies and cumulative frequencies in symbol order."""
    f = integer_table(sharpen(order_stat_probs(M, n, values=values), alpha))
    c = np.zeros(M, np.int64)
    for m in range(1, M):
        c[m] = c[m - 1] + f[m - 1]
    return f, c


def rate_table(f):
    """r_fx[m] = rne(-log2(f_m / 256) * 2^16) as int64 (Algorithm 1 rates)."""
    f = np.asarray(f, np.float64)
    return np.rint((float(PROB_BITS) - np.log2(f)) * float(1 << RATE_FRAC_BITS)).astype(np.int64)


def budget_fx(container_bytes):
    """B = 8C - sigma bits (Eq. 3), in the same fixed point as r_fx."""
    return (8 * int(container_bytes) - SIGMA_BITS) << RATE_FRAC_BITS


def _fp32_pow2_frac(k):
    """Correctly rounded fp32 value of 2^(k/512), 0 <= k < 512, exactly.

    With y_j = 1 + j 2^-23, find j with y_j <= 2^(k/512) < y_{j+1} by comparing
    512th powers as integers, then round to the nearer end (2^(k/512) is
    irrational for 0 < k < 512, so no exact ties)."""
    if k == 0:
        return np.float32(1.0)
    rhs = 1 << (k + 23 * 512)                 # 2^k * (2^23)^512
    j = int((2.0 ** (k / 512.0) - 1.0) * (1 << 23))
    while (j + (1 << 23)) ** 512 > rhs:
        j -= 1
    while (j + 1 + (1 << 23)) ** 512 <= rhs:
        j += 1
    # midpoint (2^24 + 2j + 1) / 2^24: compare 2^k * 2^(24*512) with mid^512
    if (1 << (k + 24 * 512)) < ((1 << 24) + 2 * j + 1) ** 512:
        jj = j
    else:
        jj = j + 1
    return np.float32(1.0 + jj / float(1 << 23))


def lambda_table():
    """E[k] = RN32(2^(k/512)), k = 0..511 (float32 array)."""
    return np.array([_fp32_pow2_frac(k) for k in range(512)], np.float32)


def decode_table(f, c):
    """The 256-entry table of Algorithm 2: T[z] = (m, f_m, z - c_m)."""
    f = np.asarray(f, np.int64)
    c = np.asarray(c, np.int64)
    sym = np.zeros(256, np.int64)
    for m in range(len(f)):
        sym[c[m]:c[m] + f[m]] = m
    return sym, f[sym], np.arange(256) - c[sym]
