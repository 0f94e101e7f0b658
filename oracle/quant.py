"""FitMinMax, Drift, Refit and the per-stream encoder of Algorithm 1.

Follows [D-Quant] §4.2 Eq. (4) (token-wise affine grid: s = (max-min)/(M-1),
o = min), §4.3 Eqs. (5)-(6) (rate-constrained assignment solved through the
Lagrangian sum D_i(m_i) + lambda r(m_i)), and Appendix A, Algorithm 1 (fit,
drift, least-squares refit, FP16 rounding of s and o, a second drift against
the FP16 grid, rANS; drift bisects log2 lambda between hi = log2(8 (max D -
min D)) and hi - 40 in T = 12 steps and returns the assignment at 2^hi).

Readings (the page leaves the arithmetic open; these fix it):
  * D_im = RN(delta^2), delta = RN(x_i - rec_m), rec_m = RN(o + RN(s m)),
    all float32.  The objective is RN(D_im + RN(lambda r_m)) in float32, with
    r_m = r_fx[m] / 2^16 (exact in float32).  m_i is the lowest index that
    attains the minimum over all M levels.
  * The rate test is the exact integer comparison sum_i r_fx[m_i] <= B_fx.
  * hi = ceil(log2(8 Delta)) exactly (from the binary exponent), where
    Delta = RN(max D - min D); lambda runs on a grid of 1/512 in log2, so a
    grid point u is lambda = ldexp(E[u mod 512], floor(u / 512)); the
    bisection starts from lo = 512 (hi - 40), hi = 512 hi and, because the
    width 40 * 512 = 5 * 2^12, every midpoint is an integer.
  * If 8 Delta == 0 (all distortions equal, e.g. s == 0) every symbol takes the
    cheapest level (lowest index of the smallest rate) and no bisection runs.
  * If no tested lambda was feasible the assignment at 2^hi is evaluated; if
    that is infeasible too, every symbol takes the cheapest level (a
    "fallback"; the plan guarantees n * min r_fx <= B_fx, so it always fits).
  * Refit: least squares of x on [1, v_m] in float64 (v_m = m for affine
    levels).  S1 = sum v_m, S2 = sum v_m^2, Sx = sum x_i and Smx = sum v_m x_i
    are float64 sums in a fixed order (S1, S2 are exact for affine levels): the n values are split into 64 contiguous chunks of
    ceil(n/64) (chunk l holds i in [l q, (l+1) q)), each chunk is summed from
    +0.0 in increasing i, and the 64 partial sums are combined by six
    butterfly rounds p_l <- p_l + p_(l xor k), k = 32, 16, 8, 4, 2, 1.
    den = RN(n S2) - RN(S1 S1); if den == 0 then s' = s, o' = (Sx - s S1) / n, else
    s' = (n Smx - S1 Sx) / den, o' = (Sx - s' S1) / n (each step one float64
    operation).  If s' < 0 or anything is not finite, (s', o') = (s, o).
    The stored metadata is fp16(fp32(s')), fp16(fp32(o')).
"""

import numpy as np

from .model import budget_fx, RATE_FRAC_BITS

F32 = np.float32
F64 = np.float64

BISECT_STEPS = 12     # T in Algorithm 1
BRACKET_LOG2 = 40     # lo = hi - 40 in Algorithm 1
GRID = 512            # lambda grid points per octave


def fit_minmax(x, levels):
    """Eq. (4): s = (max - min) / (M - 1), o = min (float32, per row).

    A zero extreme is taken as +0 (min + 0 in round-to-nearest), so the sign
    of a zero offset never depends on how a -0/+0 tie is resolved."""
    x = np.asarray(x, F32)
    mn = x.min(axis=1) + F32(0.0)
    mx = x.max(axis=1) + F32(0.0)
    s = (mx - mn) / F32(levels - 1)
    return s.astype(F32), mn.astype(F32)


def _distortion(x, s, o, levels, vals=None):
    lev = np.arange(levels, dtype=F32) if vals is None else np.asarray(vals, F32)
    rec = o[:, None] + s[:, None] * lev[None, :]
    delta = x[:, :, None] - rec[:, None, :]
    return delta * delta                                  # [N, n, M] float32


def _assign(D, rate_f32, r_fx, u, E):
    """argmin_m RN(D_im + RN(lambda(u) r_m)) and the exact integer rate."""
    lam = np.ldexp(E[u & (GRID - 1)], (u >> 9).astype(np.int32))
    lr = lam[:, None] * rate_f32[None, :]
    obj = D + lr[:, None, :]
    m = np.argmin(obj, axis=2)                            # first minimum
    return m, r_fx[m].sum(axis=1)


def drift(x, s, o, r_fx, B_fx, E, trace=None, vals=None):
    """Drift(x, s, o, r, B) of Algorithm 1 for every row of x.

    B_fx is the budget in rate fixed point (``model.budget_fx(C)``).  If
    ``trace`` is a list, the lambda grid point of every evaluation is appended.
    ``vals`` are the level values (float32; None: v_m = m), so that
    rec_m = RN(o + RN(s v_m)).
    Returns (m [N, n] int64, fallback [N] bool)."""
    x = np.asarray(x, F32)
    s = np.asarray(s, F32)
    o = np.asarray(o, F32)
    r_fx = np.asarray(r_fx, np.int64)
    N, n = x.shape
    M = len(r_fx)
    rate_f32 = (r_fx.astype(F64) / float(1 << RATE_FRAC_BITS)).astype(F32)
    m_star = int(np.argmin(r_fx))
    D = _distortion(x, s, o, M, vals)
    y = (D.max(axis=(1, 2)) - D.min(axis=(1, 2))) * F32(8)
    if not np.all(np.isfinite(y)):
        raise ValueError("distortion range is not finite")
    m = np.full((N, n), m_star, np.int64)
    fallback = np.zeros(N, bool)
    idx = np.nonzero(y > 0)[0]
    if len(idx):
        frac, e = np.frexp(y[idx])
        hi0 = np.where(frac == F32(0.5), e - 1, e).astype(np.int64)
        lo_u = GRID * (hi0 - BRACKET_LOG2)
        hi_u = GRID * hi0
        Dl = D[idx]
        best = np.full((len(idx), n), m_star, np.int64)
        moved = np.zeros(len(idx), bool)
        for _ in range(BISECT_STEPS):
            mid = (lo_u + hi_u) // 2
            if trace is not None:
                trace.append(mid.copy())
            mm, R = _assign(Dl, rate_f32, r_fx, mid, E)
            ok = R <= B_fx
            hi_u = np.where(ok, mid, hi_u)
            lo_u = np.where(ok, lo_u, mid)
            best[ok] = mm[ok]
            moved |= ok
        rest = np.nonzero(~moved)[0]
        if len(rest):
            if trace is not None:
                trace.append(hi_u[rest].copy())
            mm, R = _assign(Dl[rest], rate_f32, r_fx, hi_u[rest], E)
            ok = R <= B_fx
            best[rest[ok]] = mm[ok]
            best[rest[~ok]] = m_star
            fallback[idx[rest[~ok]]] = True
        m[idx] = best
    return m, fallback


def lane_sum_f64(v):
    """Sum each row of float64 v [N, n] in the fixed 64-chunk butterfly order."""
    v = np.asarray(v, F64)
    N, n = v.shape
    q = -(-n // 64)
    p = np.zeros((N, 64), F64)
    lanes = np.arange(64)
    for r in range(q):
        i = lanes * q + r
        ok = i < n
        p[:, lanes[ok]] = p[:, lanes[ok]] + v[:, i[ok]]
    for k in (32, 16, 8, 4, 2, 1):
        p = p + p[:, lanes ^ k]
    return p[:, 0]


def refit_f64(x, m, s, o, vals=None):
    """Least-squares (s', o') of x on [1, v_m] in float64, with the guard.

    The level sums S1 = sum v_m, S2 = sum v_m^2 use the same fixed order as the
    other sums; with affine levels they are exact integers, and so is
    den = RN(n S2) - RN(S1 S1) (below 2^53)."""
    x = np.asarray(x, F32)
    m = np.asarray(m, np.int64)
    N, n = x.shape
    vd = (m.astype(F64) if vals is None else np.asarray(vals, F32).astype(F64)[m])
    S1d = lane_sum_f64(vd)
    S2d = lane_sum_f64(vd * vd)
    xd = x.astype(F64)
    Sx = lane_sum_f64(xd)
    Smx = lane_sum_f64(vd * xd)
    nd = F64(n)
    den = nd * S2d - S1d * S1d
    s64 = np.asarray(s, F32).astype(F64)
    o64 = np.asarray(o, F32).astype(F64)
    with np.errstate(all="ignore"):
        flat = den == 0
        den_d = np.where(flat, 1, den).astype(F64)
        s_new = np.where(flat, s64, (nd * Smx - S1d * Sx) / den_d)
        o_new = (Sx - s_new * S1d) / nd
    bad = ~(s_new >= 0) | ~np.isfinite(s_new) | ~np.isfinite(o_new)
    return np.where(bad, s64, s_new), np.where(bad, o64, o_new)


def refit(x, m, s, o, vals=None):
    """Refit (s, o) to the assignment m, then round to fp16 via fp32.

    Returns (s16, o16) as float16 arrays."""
    s_new, o_new = refit_f64(x, m, s, o, vals)
    with np.errstate(over="ignore"):
        s16 = s_new.astype(F32).astype(np.float16)
        o16 = o_new.astype(F32).astype(np.float16)
    if not (np.all(np.isfinite(s16)) and np.all(np.isfinite(o16))):
        raise ValueError("scale or offset overflows fp16")
    return s16, o16


def nearest_levels(x, s, o, levels, vals=None):
    """argmin_m D_im (lowest index on ties): the lambda -> 0 assignment."""
    D = _distortion(np.asarray(x, F32), np.asarray(s, F32), np.asarray(o, F32), levels, vals)
    return np.argmin(D, axis=2)


def encode_streams_alg1(x, levels, f, c, r_fx, container_bytes, E, vals=None):
    """Algorithm 1 for each row of x (already rotated and, for keys, centred).

    Returns a dict with the containers [N, C] (uint8), s16/o16 (float16 [N]),
    symbols m [N, n], per-pass fallback flags and the count of symbols that
    differ from nearest rounding on the final grid."""
    from .rans import rans_encode
    x = np.asarray(x, F32)
    s, o = fit_minmax(x, levels)
    B_fx = budget_fx(container_bytes)
    m1, fb1 = drift(x, s, o, r_fx, B_fx, E, vals=vals)
    s16, o16 = refit(x, m1, s, o, vals)
    s2 = s16.astype(F32)
    o2 = o16.astype(F32)
    m2, fb2 = drift(x, s2, o2, r_fx, B_fx, E, vals=vals)
    cont, k = rans_encode(m2, f, c, container_bytes)
    changed = int((nearest_levels(x, s2, o2, levels, vals) != m2).sum())
    return {"cont": cont, "s16": s16, "o16": o16, "m": m2, "payload": k,
            "fallback1": fb1, "fallback2": fb2, "changed": changed}
