"""Per-element comparison metric for device results (test infrastructure).

The bars: max relative error per element <= 8e-3 where the output is bf16
(MATCH, and wide-internal with bf16 output), <= 1e-4 for wide-internal with
float32 output.  A plain ``|y - r| / |r|`` is undefined at ``r = 0`` and
meaningless where the gate or up dot product has cancelled far below its
terms, so the denominator is floored:

    err_i = |y_i - r_i| / max(|r_i|, tau_i, tau_0)
    tau_i = 2^-4 * ( |silu(g_i)| * nu_u,i + |silu'(g_i) * u_i| * nu_g,i )
    tau_0 = 2^-24 * RMS(r)

``nu = sqrt(sum_k (x_k w_k)^2)`` is the cancellation-free scale of a dot
product; ``tau_i`` is first-order error propagation of a gate/up error of
1/16 of that scale.  Where no cancellation happened the floor does not bind and
the test is plain relative error.

In MATCH the gate and up are rounded to bf16 before the nonlinearity.  Where
the exact value lies within ``eta * nu`` (eta = 2^-12) of a bf16 rounding
midpoint, a correct float32 accumulation may round to either neighbour; both
are admissible, and the candidate nearest the device value is used.

Binary16 activations (the oracle dict's ``act`` = 1): the 16-bit output and
MATCH's gate/up rounding are binary16, and the bar for a binary16 output is
1e-3 -- two binary16 half-ulps (2^-11 each), as 8e-3 is two bf16 half-ulps
(2^-8) rounded up: the one rounding at the store plus float32 error.  float32
output keeps 1e-4.  An output below its type's normal range is rounded to
that type's subnormal quantum (binary16: 2^-24, bf16: 2^-133, float32:
2^-149), an absolute error up to half of it on top of the relative error
of the steps before; so the denominator gains ``quantum / (2 tol)``, which
admits exactly that rounding beside the relative bar (and is negligible for
any output in the type's normal range).
"""
from __future__ import annotations

import numpy as np

from . import bf16_rne, bf16_value, f16_rne, f16_value, silu

TOL = {0: 8e-3, 1: 1e-4, 2: 8e-3}
TOL_F16 = {0: 1e-3, 1: 1e-4, 2: 1e-3}
ETA = 2.0 ** -12
FLOOR = 2.0 ** -4
TAU0 = 2.0 ** -24


def _sigmoid(t):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-t))


def silu_prime(t):
    s = _sigmoid(t)
    return s * (1.0 + t * (1.0 - s))


def _rounding(act):
    return (f16_rne, f16_value) if act else (bf16_rne, bf16_value)


def output_quantum(mode, act):
    """The smallest subnormal of the output type: float32 in mode 1, else the
    16-bit activation type."""
    if mode == 1:
        return 2.0 ** -149
    return 2.0 ** -24 if act else 2.0 ** -133


def bf16_candidates(v, nu, eta=ETA, act=0):
    """(primary, alternative) bf16 (act 1: binary16) roundings of float64 ``v``
    as float64.

    primary = RNE(v).  alternative = the other neighbour of ``v`` when ``v``
    lies within ``eta * nu`` of the midpoint between the two; otherwise it
    equals primary."""
    rne, value = _rounding(act)
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    sign = np.where(np.signbit(v), -1.0, 1.0)
    pb = rne(a).astype(np.int64)
    pv = value(pb.astype(np.uint16))
    above = pv > a
    ob = np.where(above, np.maximum(pb - 1, 0), pb + 1)
    ov = value(ob.astype(np.uint16))
    exact = pv == a
    mid = 0.5 * (pv + ov)
    admissible = (~exact) & (np.abs(a - mid) <= eta * np.asarray(nu, dtype=np.float64))
    alt = np.where(admissible, ov, pv)
    return sign * pv, sign * alt


def reference_values(o, mode):
    """Primary reference r and its gate/up (rounded in MATCH to the activation type)."""
    g, u = o["g"], o["u"]
    if mode == 0:
        rne, value = _rounding(o.get("act", 0))
        g = value(rne(g))
        u = value(rne(u))
    return silu(g) * u, g, u


def evaluate(y, o, mode, eta=ETA):
    """Compare device output ``y`` (any float dtype, same element order as the
    oracle dict ``o``) against the oracle.  Returns a dict of statistics with
    ``ok`` set when the bar of ``mode`` holds."""
    y = np.asarray(y, dtype=np.float64).reshape(-1)
    act = int(o.get("act", 0))
    tol = (TOL_F16 if act else TOL)[mode]
    g, u = o["g"].reshape(-1), o["u"].reshape(-1)
    nug, nuu = o["nu_g"].reshape(-1), o["nu_u"].reshape(-1)
    r0, gp, up = reference_values({"g": g, "u": u, "act": act}, mode)
    if mode == 0:
        g_a, g_b = bf16_candidates(g, nug, eta, act)
        u_a, u_b = bf16_candidates(u, nuu, eta, act)
        cands = [silu(gc) * uc for gc in (g_a, g_b) for uc in (u_a, u_b)]
        dist = np.stack([np.abs(y - c) for c in cands])
        pick = np.argmin(dist, axis=0)
        r = np.choose(pick, cands)
    else:
        r = r0
    tau = FLOOR * (np.abs(silu(gp)) * nuu + np.abs(silu_prime(gp) * up) * nug)
    rms = float(np.sqrt(np.mean(r0 * r0))) if r0.size else 0.0
    tau0 = TAU0 * rms
    denom = np.maximum(np.maximum(np.abs(r), tau), tau0) + output_quantum(mode, act) / 2.0 / tol
    diff = np.abs(y - r)
    finite = np.isfinite(y)
    with np.errstate(divide="ignore", invalid="ignore"):
        err = np.where(denom > 0, diff / np.where(denom > 0, denom, 1.0),
                       np.where(diff == 0, 0.0, np.inf))
    err = np.where(finite, err, np.inf)
    n = y.size
    worst = int(np.argmax(err)) if n else -1
    stats = {
        "n": n,
        "max_err": float(err[worst]) if n else 0.0,
        "worst_index": worst,
        "floor_fraction": float(np.mean(np.maximum(tau, tau0) > np.abs(r))) if n else 0.0,
        "max_abs_over_rms": float(np.max(diff) / rms) if (n and rms > 0) else 0.0,
        "nonfinite": int(np.sum(~finite)),
        "tol": tol,
    }
    stats["ok"] = bool(n == 0 or (stats["nonfinite"] == 0 and stats["max_err"] <= tol))
    return stats


LINEAR_TOL = {0: 8e-3, 1: 1e-4}   # bf16 output, float32 output


def evaluate_linear(y, r, nu, out_mode, eta=ETA):
    """Compare a device linear ``y = x W^T`` against the oracle's float64 sums
    ``r`` and their scales ``nu``.  The same metric with the floor of a single
    dot product, ``tau_i = 2^-4 * nu_i``; for bf16 output both roundings of a
    sum within ``eta * nu`` of a bf16 midpoint are admissible."""
    y = np.asarray(y, dtype=np.float64).reshape(-1)
    r0 = np.asarray(r, dtype=np.float64).reshape(-1)
    nu = np.asarray(nu, dtype=np.float64).reshape(-1)
    if out_mode == 0:
        a, b = bf16_candidates(r0, nu, eta)
        ref = np.where(np.abs(y - a) <= np.abs(y - b), a, b)
    else:
        ref = r0
    rms = float(np.sqrt(np.mean(r0 * r0))) if r0.size else 0.0
    denom = np.maximum(np.maximum(np.abs(ref), FLOOR * nu), TAU0 * rms)
    diff = np.abs(y - ref)
    finite = np.isfinite(y)
    with np.errstate(divide="ignore", invalid="ignore"):
        err = np.where(denom > 0, diff / np.where(denom > 0, denom, 1.0),
                       np.where(diff == 0, 0.0, np.inf))
    err = np.where(finite, err, np.inf)
    n = y.size
    worst = int(np.argmax(err)) if n else -1
    stats = {"n": n, "max_err": float(err[worst]) if n else 0.0, "worst_index": worst,
             "nonfinite": int(np.sum(~finite)), "tol": LINEAR_TOL[out_mode],
             "max_abs_over_rms": float(np.max(diff) / rms) if (n and rms > 0) else 0.0}
    stats["ok"] = bool(n == 0 or (stats["nonfinite"] == 0 and stats["max_err"] <= LINEAR_TOL[out_mode]))
    return stats


# The whole MLP's hidden tensor is the forward's bf16 output, which may differ
# from the oracle's rounding by an admissible bf16 neighbour (a gate or up sum
# near a rounding midpoint, the final rounding of silu * up) at a small
# fraction of elements.  Each such element moves the down projection by at
# most 2^-6 |hidden_i wd_i|; with random signs the sum moves by well under
# 2^-7 nu, which is the allowance added to the output's own bar.
HIDDEN_SLACK = 2.0 ** -7


def evaluate_mlp(y, r, nu, out_mode, eta=ETA):
    """Compare a device whole-MLP output with the oracle's float64 result ``r``
    and the down projection's scale ``nu``: pass iff every element satisfies
    ``|y - ref| <= tol * max(|ref|, 2^-4 nu, tau_0) + 2^-7 nu`` (tol the
    linear's bar by output type; for bf16 output both roundings of a value
    within ``eta * nu`` of a midpoint are admissible).  ``max_ratio`` is the
    largest ``|y - ref|`` over its allowance (pass iff <= 1)."""
    y = np.asarray(y, dtype=np.float64).reshape(-1)
    r0 = np.asarray(r, dtype=np.float64).reshape(-1)
    nu = np.asarray(nu, dtype=np.float64).reshape(-1)
    if out_mode == 0:
        a, b = bf16_candidates(r0, nu, eta)
        ref = np.where(np.abs(y - a) <= np.abs(y - b), a, b)
    else:
        ref = r0
    rms = float(np.sqrt(np.mean(r0 * r0))) if r0.size else 0.0
    allow = LINEAR_TOL[out_mode] * np.maximum(np.maximum(np.abs(ref), FLOOR * nu), TAU0 * rms) + HIDDEN_SLACK * nu
    diff = np.abs(y - ref)
    finite = np.isfinite(y)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(allow > 0, diff / np.where(allow > 0, allow, 1.0), np.where(diff == 0, 0.0, np.inf))
    ratio = np.where(finite, ratio, np.inf)
    n = y.size
    worst = int(np.argmax(ratio)) if n else -1
    stats = {"n": n, "max_ratio": float(ratio[worst]) if n else 0.0, "worst_index": worst,
             "nonfinite": int(np.sum(~finite)), "tol": LINEAR_TOL[out_mode], "slack": HIDDEN_SLACK,
             "max_abs_over_nu": float(np.max(diff / np.maximum(nu, 1e-300))) if n else 0.0}
    stats["ok"] = bool(n == 0 or (stats["nonfinite"] == 0 and stats["max_ratio"] <= 1.0))
    return stats
