"""Pins of the oracle's binary16-activation form (x, scales and biases as IEEE
float16, the pages' second activation type) against facts that do not come
from the oracle itself: numpy's own float16 decoding and rounding, an exact
rational brute force with its own binary16 decoder, problems whose values are
the same in both activation types, and planted errors that the metric's
binary16 bar must catch."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import compare, exact
from synth import make_custom, to_bf16_bits, to_f16_bits

SPECS = [(4, 32), (4, 64), (8, 32), (8, 128), (2, 64)]


def _rel_to_scale(a, b, scale):
    return abs(a - b) / max(scale, 1e-300)


# ------------------------------------------------------------ conversions --

def test_f16_value_every_bit_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.f16_value(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[0x7C00] == np.inf and got[0xFC00] == -np.inf
    assert got[0x0001] == 2.0 ** -24 and got[0x7BFF] == 65504.0


def test_f16_rne_matches_numpy():
    rng = np.random.default_rng(5)
    mags = np.ldexp(rng.uniform(1.0, 2.0, 20000), rng.integers(-30, 18, 20000))
    vals = np.concatenate([mags, -mags])
    # exact midpoints between neighbours (ties go to the even one), in the
    # normal and the subnormal range, and the overflow boundary
    f = np.arange(1, 0x7BFF, 97, dtype=np.uint16).view(np.float16).astype(np.float64)
    nxt = (np.arange(1, 0x7BFF, 97, dtype=np.uint16) + 1).view(np.float16).astype(np.float64)
    mids = (f + nxt) / 2
    edges = np.array([65504.0, 65519.99, 65520.0, 65535.0, 65536.0, 1e9, 2.0 ** -25, 2.0 ** -26,
                      3 * 2.0 ** -26, 2.0 ** -14 - 2.0 ** -26, 5e-324, 0.0, -0.0])
    vals = np.concatenate([vals, mids, -mids, edges, -edges])
    got = oracle.f16_rne(vals)
    with np.errstate(over="ignore"):
        ref = vals.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def test_f16_exact_decoder_agrees():
    bits = [b for b in range(1 << 16) if ((b >> 10) & 0x1F) != 0x1F]
    vals = oracle.f16_value(np.array(bits, dtype=np.uint16))
    for b, v in zip(bits[::7], vals[::7]):
        assert exact.f16_exact(b) == Fraction(float(v))


# ------------------------------------------------------------ the forward --

@pytest.mark.parametrize("bits,gs", SPECS)
def test_f16_oracle_matches_exact_rationals(bits, gs):
    M, H, I = 3, 128, 4
    p = make_custom(M, H, I, bits, gs, bits, gs, seed=bits * 11 + gs, act="f16")
    o = oracle.swiglu_full(p, mode=1, nthreads=1)
    assert o["act"] == 1
    xg = [list(r) for r in p.x]
    ex_g = exact.qmm_exact(xg, p.wg, p.sg, p.bg, M, H, I, bits, gs, act="f16")
    ex_u = exact.qmm_exact(xg, p.wu, p.su, p.bu, M, H, I, bits, gs, act="f16")
    for m in range(M):
        for n in range(I):
            assert _rel_to_scale(o["g"][m, n], float(ex_g[m][n]), o["nu_g"][m, n]) <= 1e-14
            assert _rel_to_scale(o["u"][m, n], float(ex_u[m][n]), o["nu_u"][m, n]) <= 1e-14
    # reading the same bit patterns as bf16 gives other values: the type is honoured
    q = make_custom(M, H, I, bits, gs, bits, gs, seed=bits * 11 + gs, act="f16")
    q.act = "bf16"
    assert not np.allclose(oracle.swiglu_full(q, mode=1, nthreads=1)["g"], o["g"])


def test_same_values_in_both_types_give_the_same_sums():
    """Values with 8 significant bits in binary16's range are the same number
    as bf16 and as binary16: both activation types must give identical
    gate/up sums and, in the wide modes, identical hidden values."""
    rng = np.random.default_rng(9)
    M, H, I, gs = 4, 256, 6, 64
    p = make_custom(M, H, I, 4, gs, 4, gs, seed=3)

    def common(shape, lo, hi):
        v = np.ldexp(rng.integers(128, 256, shape).astype(np.float64), rng.integers(lo, hi, shape) - 7)
        return (v * rng.choice([-1.0, 1.0], shape)).astype(np.float32)

    x, sg, su = common((M, H), -6, 4), np.abs(common((I, H // gs), -9, -5)), np.abs(common((I, H // gs), -9, -5))
    bg, bu = common((I, H // gs), -6, -2), common((I, H // gs), -6, -2)
    import copy
    pb, pf = copy.deepcopy(p), copy.deepcopy(p)
    pb.x, pb.sg, pb.su, pb.bg, pb.bu = (to_bf16_bits(a) for a in (x, sg, su, bg, bu))
    pf.x, pf.sg, pf.su, pf.bg, pf.bu = (to_f16_bits(a) for a in (x, sg, su, bg, bu))
    pf.act = "f16"
    for mode in (1, 2):
        ob, of = oracle.swiglu_full(pb, mode, 1), oracle.swiglu_full(pf, mode, 1)
        for k in ("g", "u", "nu_g", "nu_u", "h"):
            assert np.array_equal(ob[k], of[k]), (mode, k)


def test_f16_match_rounds_gate_and_up_to_binary16():
    p = make_custom(5, 256, 40, 4, 64, 8, 32, seed=21, act="f16")
    wide = oracle.swiglu_full(p, 1, 1)
    match = oracle.swiglu_full(p, 0, 1)
    g16 = wide["g"].astype(np.float16).astype(np.float64)
    u16 = wide["u"].astype(np.float16).astype(np.float64)
    ref = g16 / (1.0 + np.exp(-g16)) * u16
    assert np.allclose(match["h"], ref, rtol=1e-14, atol=0.0)
    assert not np.array_equal(match["h"], wide["h"])


# ---------------------------------------------------------------- metric --

def test_f16_metric_bar():
    p = make_custom(6, 256, 96, 4, 64, seed=2, act="f16")
    for mode in (0, 1, 2):
        o = oracle.swiglu_full(p, mode)
        r, _, _ = compare.reference_values(o, mode)
        st = compare.evaluate(r, o, mode)
        assert st["ok"] and st["max_err"] == 0.0 and st["tol"] == compare.TOL_F16[mode]
    o = oracle.swiglu_full(p, 2)
    r = compare.reference_values(o, 2)[0].reshape(-1)
    big = np.argmax(np.abs(r))
    for rel, ok in ((4e-4, True), (1.5e-3, False)):
        y = r.copy()
        y[big] *= 1.0 + rel
        assert compare.evaluate(y, o, 2)["ok"] == ok, rel


def test_f16_candidates_near_midpoint():
    # 1 + 2^-11 is the binary16 midpoint between 1 and 1 + 2^-10
    v = np.array([1.0 + 2.0**-11 + 2.0**-24, 1.0 + 2.0**-12])
    pv, alt = compare.bf16_candidates(v, np.array([2.0**-4, 2.0**-4]), act=1)   # eta nu = 2^-16
    assert pv[0] == 1.0 + 2.0**-10 and alt[0] == 1.0
    assert pv[1] == 1.0 and alt[1] == 1.0


@pytest.mark.parametrize("kind", ["no_bias", "wrong_group", "k_tail", "swap_gate_up"])
def test_f16_metric_catches_planted_mistakes(kind):
    import copy
    p = make_custom(6, 256, 96, 4, 64, seed=4, act="f16")
    q = copy.deepcopy(p)
    if kind == "no_bias":
        q.bg = np.zeros_like(q.bg)
    elif kind == "wrong_group":
        q.sg = np.roll(q.sg, 1, axis=1)
    elif kind == "k_tail":
        q.x = q.x.copy()
        q.x[:, -32:] = 0
    else:
        q.wg, q.wu, q.sg, q.su, q.bg, q.bu = q.wu, q.wg, q.su, q.sg, q.bu, q.bg
    for mode in (0, 1):
        o = oracle.swiglu_full(p, mode)
        bad = compare.reference_values(oracle.swiglu_full(q, mode), mode)[0]
        st = compare.evaluate(bad.astype(np.float32), o, mode)
        assert not st["ok"] and st["max_err"] > 50 * compare.TOL_F16[mode], (kind, mode, st)

