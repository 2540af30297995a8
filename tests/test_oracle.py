"""Pins of the CPU oracle against facts that do not come from the oracle itself:
hand-derived packed words and roundings, exact rational brute force, integer
special cases that reduce to an integer matmul, closed forms of the SwiGLU
composition, and planted mistakes that the comparison metric must catch."""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import compare, exact
from synth import (CONFIGS, bf16_bits_to_f32, make_custom, make_down, make_problem, make_residual,
                   pack_codes, to_bf16_bits)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SPECS = [(4, 32), (4, 64), (4, 128), (8, 32), (8, 64), (8, 128), (2, 32), (2, 64)]


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield [p.strip() for p in line.split("|")]


# ---------------------------------------------------------------- layout ----

def test_pack_words_closed_form():
    for bits_s, codes_s, word_s in _golden_lines("pack_words.txt"):
        bits = int(bits_s)
        codes = np.array([int(c) for c in codes_s.split()], dtype=np.uint8)[None, :]
        word = int(word_s, 16)
        assert int(pack_codes(codes, bits)[0, 0]) == word
        back = oracle.unpack(np.array([[word]], dtype=np.uint32), 1, codes.shape[1], bits)
        assert np.array_equal(back, codes)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_pack_unpack_roundtrip(bits):
    rng = np.random.default_rng(bits)
    codes = rng.integers(0, 1 << bits, size=(37, 256), dtype=np.uint8)
    W = pack_codes(codes, bits)
    assert W.shape == (37, 256 * bits // 32)
    assert np.array_equal(oracle.unpack(W, 37, 256, bits), codes)
    # and the other direction: random words survive unpack -> pack
    words = rng.integers(0, 2**32, size=(5, 256 * bits // 32), dtype=np.uint64).astype(np.uint32)
    assert np.array_equal(pack_codes(oracle.unpack(words, 5, 256, bits), bits), words)


# ------------------------------------------------------------- rounding ----

def test_bf16_rne_hand_cases():
    for hx, bits_s, note in _golden_lines("bf16_rne_cases.txt"):
        v = float.fromhex(hx)
        got = int(oracle.bf16_rne(np.array([v]))[0])
        assert got == int(bits_s, 16), (hx, note, hex(got))


def test_bf16_rne_matches_torch_on_float32_values():
    """On values that are exactly float32 the direct rounding must agree with
    torch's float32 -> bfloat16 cast (a library routine)."""
    rng = np.random.default_rng(123)
    pats = rng.integers(0, 2**32, size=1 << 21, dtype=np.uint64).astype(np.uint32)
    # every exponent with ties and near-ties in the low 16 bits
    exps = np.arange(0, 255, dtype=np.uint32) << np.uint32(23)
    lows = np.array([0x0000, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x18000, 0x10000], dtype=np.uint32)
    extra = (exps[:, None] | lows[None, :]).reshape(-1)
    pats = np.concatenate([pats, extra, extra | np.uint32(0x80000000),
                           np.array([0x7F7FFFFF, 0x7F7F8000, 0x00000001, 0x80000000], dtype=np.uint32)])
    f = pats.view(np.float32)
    f = f[np.isfinite(f)]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_rne(f.astype(np.float64))
    assert np.array_equal(got, ref)


def test_silu_closed_forms():
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    t = np.linspace(-30, 30, 1201)
    d = oracle.silu(t) - oracle.silu(-t)
    np.testing.assert_allclose(d, t, rtol=1e-14, atol=1e-14)
    # sigma(ln 3) = 3/4, so silu(ln 3) = 0.75 ln 3
    assert abs(oracle.silu(np.array([math.log(3.0)]))[0] - 0.75 * math.log(3.0)) < 1e-15
    # very negative inputs underflow to -0/0 rather than NaN
    assert np.all(np.isfinite(oracle.silu(np.array([-800.0, -1e6, 800.0]))))


# ------------------------------------------------ exact brute force --------

def _rel_to_scale(a, b, scale):
    return np.abs(np.asarray(a, dtype=np.float64) - np.asarray(b, dtype=np.float64)) / np.maximum(scale, 1e-300)


@pytest.mark.parametrize("bits,gs", SPECS)
@pytest.mark.parametrize("H", [32, 64, 128])
def test_oracle_matches_exact_rationals(bits, gs, H):
    if H % gs:
        pytest.skip("H must be a multiple of gs")
    M, I = 3, 4
    p = make_custom(M, H, I, bits, gs, bits, gs, seed=H + bits * 7 + gs)
    o = oracle.swiglu_full(p, mode=1, nthreads=1)
    xg = [list(r) for r in p.x]
    ex_g = exact.qmm_exact(xg, p.wg, p.sg, p.bg, M, H, I, bits, gs)
    ex_u = exact.qmm_exact(xg, p.wu, p.su, p.bu, M, H, I, bits, gs)
    for m in range(M):
        for n in range(I):
            assert _rel_to_scale(o["g"][m, n], float(ex_g[m][n]), o["nu_g"][m, n]) <= 1e-14
            assert _rel_to_scale(o["u"][m, n], float(ex_u[m][n]), o["nu_u"][m, n]) <= 1e-14
    # the per-group decomposition reaches the same exact value
    assert exact.qmm_grouped_exact(xg, p.wg, p.sg, p.bg, M, H, I, bits, gs) == ex_g


@pytest.mark.parametrize("bits,gs", SPECS)
def test_nu_matches_exact_rationals(bits, gs):
    """The scale nu = sqrt(sum_k (x_k w_k)^2) that sets every floor of the
    comparison metric, against its exact rational value: float64 within
    1e-14 relative of the exact square root, for the gate and the up matrix."""
    M, H, I = 2, 128, 3
    p = make_custom(M, H, I, bits, gs, 8 if bits != 8 else 4, 32, seed=bits * 13 + gs)
    o = oracle.swiglu_full(p, mode=1, nthreads=1)
    xg = [list(r) for r in p.x]
    sq_g = exact.qmm_sq_exact(xg, p.wg, p.sg, p.bg, M, H, I, bits, gs)
    sq_u = exact.qmm_sq_exact(xg, p.wu, p.su, p.bu, M, H, I, p.bits_u, p.gs_u)
    for m in range(M):
        for n in range(I):
            for got, sq in ((o["nu_g"][m, n], sq_g[m][n]), (o["nu_u"][m, n], sq_u[m][n])):
                ref = math.sqrt(float(sq))
                assert ref > 0 and abs(got - ref) <= 1e-14 * ref, (got, ref)


def test_nu_single_term_closed_form():
    """With one nonzero input x_j, nu is exactly |x_j w_j| and the dot
    product is x_j w_j (no other term contributes)."""
    M, H, I = 1, 64, 5
    p = make_custom(M, H, I, 4, 32, 4, 32, seed=3)
    x = np.zeros((M, H), np.float32)
    x[0, 37] = -1.5
    p.x = to_bf16_bits(x)
    o = oracle.swiglu_full(p, mode=1, nthreads=1)
    codes = oracle.unpack(p.wg, I, H, 4)[:, 37].astype(np.float64)
    w = bf16_bits_to_f32(p.sg[:, 1]).astype(np.float64) * codes + bf16_bits_to_f32(p.bg[:, 1]).astype(np.float64)
    assert np.array_equal(o["nu_g"][0], np.abs(-1.5 * w))
    assert np.array_equal(o["g"][0], -1.5 * w)


@pytest.mark.parametrize("bits,gs", SPECS)
def test_linear_reference_matches_exact_rationals(bits, gs):
    """The quantized linear's reference (``qmm``, and ``qmm_pairs`` element by
    element) against exact rational arithmetic, with an odd output size."""
    M, H, N = 3, 128, 5
    p = make_custom(M, H, N, bits, gs, bits, gs, seed=bits * 13 + gs)
    xg = [list(r) for r in p.x]
    ex = exact.qmm_exact(xg, p.wg, p.sg, p.bg, M, H, N, bits, gs)
    y = oracle.qmm(p.x, p.wg, p.sg, p.bg, M, H, N, bits, gs)
    yp, nu = oracle.qmm_pairs(p.x, p.wg, p.sg, p.bg, M, H, N, bits, gs, nthreads=2)
    assert np.array_equal(y.reshape(-1), yp)            # the same sum in the same order
    ms, ns = np.array([2, 0, 1]), np.array([4, 3, 0])
    ys, nus = oracle.qmm_pairs(p.x, p.wg, p.sg, p.bg, M, H, N, bits, gs, ms, ns)
    assert np.array_equal(ys, y[ms, ns]) and np.array_equal(nus, nu.reshape(M, N)[ms, ns])
    for m in range(M):
        for n in range(N):
            assert _rel_to_scale(y[m, n], float(ex[m][n]), nu[m * N + n]) <= 1e-14


def test_linear_metric_catches_planted_errors():
    """The linear bar: the float64 sums pass, their bf16 and float32
    roundings pass in their modes; a 2 % error (bf16 bar 8e-3), a 0.1 %
    error (float32 bar 1e-4) or a wrong sign fails."""
    M, H, N = 4, 256, 33
    p = make_custom(M, H, N, 4, 64, 4, 64, seed=9)
    r, nu = oracle.qmm_pairs(p.x, p.wg, p.sg, p.bg, M, H, N, 4, 64)
    assert compare.evaluate_linear(r, r, nu, 0)["ok"] and compare.evaluate_linear(r, r, nu, 1)["ok"]
    rb = oracle.bf16_value(oracle.bf16_rne(r))
    assert compare.evaluate_linear(rb, r, nu, 0)["ok"]
    assert not compare.evaluate_linear(rb, r, nu, 1)["ok"]
    assert compare.evaluate_linear(r.astype(np.float32), r, nu, 1)["ok"]
    big = np.argmax(np.abs(r))
    bad = r.copy(); bad[big] *= 1.02
    assert not compare.evaluate_linear(bad, r, nu, 0)["ok"]
    bad = r.copy(); bad[big] *= 1.001
    assert not compare.evaluate_linear(bad, r, nu, 1)["ok"]
    bad = r.copy(); bad[big] = -bad[big]
    assert not compare.evaluate_linear(bad, r, nu, 1)["ok"]


# ------------------------------------------------------------- whole MLP --

@pytest.mark.parametrize("bits_d,gs_d", [(4, 64), (8, 32), (2, 128)])
def test_mlp_reference_matches_exact_rationals(bits_d, gs_d):
    """The whole MLP's down projection and residual against exact rationals,
    on the oracle's own bf16 hidden rows (the forward, pinned above, rounded):
    every output within 1e-14 of the down projection's scale; asking for a
    subset of elements gives the same values."""
    M, H, I, Ho = 2, 128, 128, 5
    p = make_custom(M, H, I, 4, 64, 8, 32, seed=gs_d + bits_d)
    wd, sd, bd = make_down(Ho, I, bits_d, gs_d, seed=7)
    res = make_residual(M, Ho, seed=8)
    y, nu, rows, hb = oracle.mlp_pairs(p, wd, sd, bd, bits_d, gs_d, Ho, res)
    assert list(rows) == list(range(M))
    assert np.array_equal(hb, oracle.bf16_rne(oracle.swiglu_full(p, 0)["h"]))
    ex = exact.qmm_exact([list(r) for r in hb], wd, sd, bd, M, I, Ho, bits_d, gs_d)
    for m in range(M):
        for n in range(Ho):
            ref = ex[m][n] + exact.bf16_exact(res[m, n])
            assert _rel_to_scale(y[m * Ho + n], float(ref), nu[m * Ho + n] + abs(float(ref))) <= 1e-14
    ms, ns = np.array([1, 0, 1]), np.array([4, 2, 0])
    ys, nus, rows2, _ = oracle.mlp_pairs(p, wd, sd, bd, bits_d, gs_d, Ho, res, ms, ns)
    assert list(rows2) == [0, 1]
    assert np.array_equal(ys, y.reshape(M, Ho)[ms, ns]) and np.array_equal(nus, nu.reshape(M, Ho)[ms, ns])


def _zero_matrix(rows, K, bits, gs, seed):
    """Constant codes q = 8 with biases -8 s: every dequantized weight is 0."""
    rng = np.random.default_rng(seed)
    codes = np.full((rows, K), 8, dtype=np.uint8)
    s = to_bf16_bits(rng.uniform(0.005, 0.02, size=(rows, K // gs)).astype(np.float32))
    b = to_bf16_bits((np.float32(-8.0) * bf16_bits_to_f32(s)).astype(np.float32))   # exact: a power of two
    return pack_codes(codes, bits), s, b


def test_mlp_closed_forms_give_the_residual():
    """Zero down weights, or a zero gate (silu(0) = 0, so the hidden tensor
    vanishes), leave exactly the residual; without a residual, exactly 0."""
    M, H, I, Ho = 3, 128, 192, 64
    p = make_custom(M, H, I, 4, 64, seed=3)
    res = make_residual(M, Ho, seed=4)
    wd, sd, bd = _zero_matrix(Ho, I, 4, 64, seed=5)
    y, nu, _, _ = oracle.mlp_pairs(p, wd, sd, bd, 4, 64, Ho, res)
    assert np.array_equal(y, bf16_bits_to_f32(res).astype(np.float64).reshape(-1)) and not nu.any()
    y0, _, _, _ = oracle.mlp_pairs(p, wd, sd, bd, 4, 64, Ho)
    assert not y0.any()
    p.wg, p.sg, p.bg = _zero_matrix(I, H, 4, 64, seed=6)
    wd, sd, bd = make_down(Ho, I, 4, 64, seed=7)
    y, nu, _, hb = oracle.mlp_pairs(p, wd, sd, bd, 4, 64, Ho, res)
    assert not (hb & 0x7FFF).any()
    assert np.array_equal(y, bf16_bits_to_f32(res).astype(np.float64).reshape(-1))


def test_mlp_metric_allows_hidden_roundings_and_catches_planted_errors():
    """The whole-MLP bar: the oracle's result with 1 % of its hidden
    elements moved to their other bf16 neighbour (ten times the rate of
    admissible roundings measured on the device) passes, rounded to bf16 or
    float32; a dropped group of the down projection, a missing residual, a
    3 % error or a wrong sign fails."""
    M, H, I, Ho = 2, 512, 2048, 256
    p = make_custom(M, H, I, 4, 64, seed=11)
    wd, sd, bd = make_down(Ho, I, 4, 64, seed=12)
    res = make_residual(M, Ho, seed=13)
    r, nu, _, hb = oracle.mlp_pairs(p, wd, sd, bd, 4, 64, Ho, res)
    rng = np.random.default_rng(14)
    moved = hb.copy()
    pick = rng.random(hb.shape) < 0.01
    nonzero = (hb & 0x7FFF) != 0
    step = np.where(rng.random(hb.shape) < 0.5, 1, -1).astype(np.int32)
    moved = np.where(pick & nonzero, (moved.astype(np.int32) + step).astype(np.uint16), moved)
    assert (moved != hb).sum() > 0.005 * hb.size
    rb = oracle.bf16_value(res).reshape(-1)
    y_moved, _ = oracle.qmm_pairs(moved, wd, sd, bd, M, I, Ho, 4, 64)
    y_moved = y_moved + rb
    assert compare.evaluate_mlp(r, r, nu, 0)["ok"] and compare.evaluate_mlp(r, r, nu, 1)["ok"]
    assert compare.evaluate_mlp(oracle.bf16_value(oracle.bf16_rne(y_moved)), r, nu, 0)["ok"]
    assert compare.evaluate_mlp(y_moved.astype(np.float32), r, nu, 1)["ok"]
    # planted errors
    sd_drop = sd.copy(); bd_drop = bd.copy()
    sd_drop[:, 5] = 0; bd_drop[:, 5] = 0                      # group 5 of every output contributes nothing
    y_drop, _ = oracle.qmm_pairs(hb, wd, sd_drop, bd_drop, M, I, Ho, 4, 64)
    y_drop = y_drop + rb
    assert not compare.evaluate_mlp(y_drop.astype(np.float32), r, nu, 1)["ok"]
    assert not compare.evaluate_mlp(oracle.bf16_value(oracle.bf16_rne(y_drop)), r, nu, 0)["ok"]
    assert not compare.evaluate_mlp(r - rb, r, nu, 0)["ok"]
    big = np.argmax(np.abs(r))
    bad = r.copy(); bad[big] *= 1.03
    assert not compare.evaluate_mlp(bad, r, nu, 0)["ok"]
    bad = r.copy(); bad[big] = -bad[big]
    assert not compare.evaluate_mlp(bad, r, nu, 1)["ok"]


@pytest.mark.parametrize("case", range(24))
def test_random_specs_and_magnitudes_against_exact(case):
    """Seeded random tiny problems -- any gate/up code widths and group
    sizes, output sizes 1-4, x scaled from 2^-10 to 2^10, scales anywhere in
    the documented exact range [2^-17, 2^8) -- against exact rationals: the
    oracle's float64 gate and up within 1e-14 of each dot product's scale."""
    rng = np.random.default_rng(1000 + case)
    bits_g, bits_u = (int(b) for b in rng.choice([2, 4, 8], 2))
    gs_g, gs_u = (int(g) for g in rng.choice([32, 64, 128], 2))
    H = int(max(gs_g, gs_u) * rng.integers(1, 3))
    M, I = int(rng.integers(1, 4)), int(rng.integers(1, 5))
    s_lo = float(2.0 ** rng.uniform(-17, 6))
    p = make_custom(M, H, I, bits_g, gs_g, bits_u, gs_u, seed=case, x_sigma=float(2.0 ** rng.uniform(-10, 10)),
                    s_lo=s_lo, s_hi=s_lo * 4, bias_mode="factor")
    o = oracle.swiglu_full(p, mode=1, nthreads=1)
    xg = [list(r) for r in p.x]
    ex_g = exact.qmm_exact(xg, p.wg, p.sg, p.bg, M, H, I, bits_g, gs_g)
    ex_u = exact.qmm_exact(xg, p.wu, p.su, p.bu, M, H, I, bits_u, gs_u)
    for m in range(M):
        for n in range(I):
            assert _rel_to_scale(o["g"][m, n], float(ex_g[m][n]), o["nu_g"][m, n]) <= 1e-14
            assert _rel_to_scale(o["u"][m, n], float(ex_u[m][n]), o["nu_u"][m, n]) <= 1e-14


def test_mixed_specs_against_exact():
    M, H, I = 2, 128, 3
    p = make_custom(M, H, I, 8, 32, 4, 64, seed=5, bias_mode="half")
    o = oracle.swiglu_full(p, mode=1, nthreads=2)
    xg = [list(r) for r in p.x]
    ex_g = exact.qmm_exact(xg, p.wg, p.sg, p.bg, M, H, I, 8, 32)
    ex_u = exact.qmm_exact(xg, p.wu, p.su, p.bu, M, H, I, 4, 64)
    for m in range(M):
        for n in range(I):
            assert _rel_to_scale(o["g"][m, n], float(ex_g[m][n]), o["nu_g"][m, n]) <= 1e-14
            assert _rel_to_scale(o["u"][m, n], float(ex_u[m][n]), o["nu_u"][m, n]) <= 1e-14


def test_integer_special_case_is_an_integer_matmul():
    """s = 1, b in {0, -8}, small-integer x: gate and up are exact integers,
    equal to an int64 matmul of codes (a library routine)."""
    rng = np.random.default_rng(9)
    M, H, I = 5, 256, 11
    for bits, gs, bval in [(4, 64, 0.0), (4, 32, -8.0), (8, 32, -8.0), (8, 128, 0.0)]:
        xi = rng.integers(-7, 8, size=(M, H))
        codes = rng.integers(0, 1 << bits, size=(I, H), dtype=np.uint8)
        one = to_bf16_bits(np.ones((I, H // gs), np.float32))
        bb = to_bf16_bits(np.full((I, H // gs), bval, np.float32))
        p = make_custom(M, H, I, bits, gs, seed=0)
        p.x = to_bf16_bits(xi.astype(np.float32))
        p.wg = p.wu = pack_codes(codes, bits)
        p.sg = p.su = one
        p.bg = p.bu = bb
        o = oracle.swiglu_full(p, mode=1)
        ref = xi.astype(np.int64) @ (codes.astype(np.int64) + int(bval)).T
        assert np.array_equal(o["g"], ref.astype(np.float64))
        assert np.array_equal(o["u"], ref.astype(np.float64))


# ------------------------------------------------------ closed forms -------

def _zero_path(p, which, bits, gs, rng):
    """Codes constant per group (c in {1,2,4,8}) and bias = -s*c exactly, so the
    dequantized weight is identically zero."""
    I, H = p.I, p.H
    c = rng.choice(np.array([1, 2, 4, 8]), size=(I, H // gs))
    codes = np.repeat(c, gs, axis=1).astype(np.uint8)
    s = bf16_bits_to_f32(getattr(p, "s" + which))
    b_bits = to_bf16_bits((-s * c).astype(np.float32))
    assert np.array_equal(bf16_bits_to_f32(b_bits), (-s * c).astype(np.float32))  # exact
    setattr(p, "w" + which, pack_codes(codes, bits))
    setattr(p, "b" + which, b_bits)


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_zero_gate_or_up_gives_zero(mode):
    rng = np.random.default_rng(77)
    for which in ("g", "u"):
        p = make_custom(4, 256, 9, 4, 64, seed=3)
        _zero_path(p, which, 4, 64, rng)
        o = oracle.swiglu_full(p, mode)
        assert np.all(o[which] == 0.0)
        assert np.all(o["h"] == 0.0)


@pytest.mark.parametrize("bits,gs", [(4, 64), (8, 32), (4, 128)])
def test_single_group_constant_codes(bits, gs):
    """H = gs with constant codes per row: gate = s'*sum(x), up = t'*sum(x),
    where s' = s*c + b and t' = s_u*c_u + b_u."""
    rng = np.random.default_rng(bits * gs)
    M, H, I = 4, gs, 6
    p = make_custom(M, H, I, bits, gs, seed=11)
    cg = rng.integers(0, 1 << bits, size=I)
    cu = rng.integers(0, 1 << bits, size=I)
    p.wg = pack_codes(np.repeat(cg[:, None], H, axis=1).astype(np.uint8), bits)
    p.wu = pack_codes(np.repeat(cu[:, None], H, axis=1).astype(np.uint8), bits)
    o = oracle.swiglu_full(p, mode=1)
    sx = bf16_bits_to_f32(p.x).astype(np.float64).sum(axis=1)
    sg, bg = (bf16_bits_to_f32(a)[:, 0].astype(np.float64) for a in (p.sg, p.bg))
    su, bu = (bf16_bits_to_f32(a)[:, 0].astype(np.float64) for a in (p.su, p.bu))
    sp = sg * cg + bg
    tp = su * cu + bu
    gate = sx[:, None] * sp[None, :]
    up = sx[:, None] * tp[None, :]
    h = gate / (1.0 + np.exp(-gate)) * up
    np.testing.assert_allclose(o["g"], gate, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(o["h"], h, rtol=1e-12, atol=1e-14)


def test_fused_equals_unfused_composition():
    p = make_custom(3, 128, 5, 4, 64, seed=21)
    o1 = oracle.swiglu_full(p, mode=1)
    o0 = oracle.swiglu_full(p, mode=0)
    g = oracle.qmm(p.x, p.wg, p.sg, p.bg, 3, 128, 5, 4, 64)
    u = oracle.qmm(p.x, p.wu, p.su, p.bu, 3, 128, 5, 4, 64)
    assert np.array_equal(o1["h"], oracle.silu(g) * u)
    gb, ub = oracle.bf16_value(oracle.bf16_rne(g)), oracle.bf16_value(oracle.bf16_rne(u))
    assert np.array_equal(o0["h"], oracle.silu(gb) * ub)


def test_pairs_equal_full():
    p = make_custom(7, 256, 33, 8, 32, 4, 64, seed=8)
    full = oracle.swiglu_full(p, mode=0)
    rng = np.random.default_rng(1)
    ms = rng.integers(0, 7, 50)
    ns = rng.integers(0, 33, 50)
    part = oracle.swiglu_pairs(p, 0, ms, ns)
    for k in ("g", "u", "nu_g", "nu_u", "h"):
        assert np.array_equal(part[k], full[k][ms, ns])


def test_oracle_rejects_bad_arguments():
    p = make_custom(2, 64, 3, 4, 64, seed=1)
    with pytest.raises(ValueError):
        oracle.swiglu_pairs(p, 0, np.array([2]), np.array([0]))
    with pytest.raises(ValueError):
        oracle.swiglu_pairs(p, 3)


# ------------------------------------------------------ the metric -------

def _emulate_f32_device(p, mode, order_seed=0):
    """A float32 computation of the method with an arbitrary summation order,
    standing in for any correct implementation (numpy/torch on the CPU)."""
    codes_g = oracle.unpack(p.wg, p.I, p.H, p.bits_g).astype(np.float64)
    codes_u = oracle.unpack(p.wu, p.I, p.H, p.bits_u).astype(np.float64)
    x = bf16_bits_to_f32(p.x).astype(np.float64)

    def proj(codes, S, B, gs):
        s = np.repeat(bf16_bits_to_f32(S).astype(np.float64), gs, axis=1)
        b = np.repeat(bf16_bits_to_f32(B).astype(np.float64), gs, axis=1)
        w = (s * codes + b).astype(np.float32)          # one float32 rounding of w
        xs = x.astype(np.float32)
        rng = np.random.default_rng(order_seed)
        perm = rng.permutation(p.H)
        acc = np.zeros((p.M, p.I), np.float32)
        for blk in np.array_split(perm, max(1, p.H // 16)):
            acc += xs[:, blk] @ w[:, blk].T
        return acc

    g = proj(codes_g, p.sg, p.bg, p.gs_g)
    u = proj(codes_u, p.su, p.bu, p.gs_u)
    if mode == 0:
        g = torch.from_numpy(g).to(torch.bfloat16).float().numpy()
        u = torch.from_numpy(u).to(torch.bfloat16).float().numpy()
    h = (g / (np.float32(1) + np.exp(-g, dtype=np.float32))) * u
    if mode in (0, 2):
        h = torch.from_numpy(h.astype(np.float32)).to(torch.bfloat16).float().numpy()
    return h.astype(np.float32)


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_metric_accepts_a_correct_float32_computation(mode):
    p = make_problem(0)
    o = oracle.swiglu_full(p, mode)
    for seed in range(3):
        y = _emulate_f32_device(p, mode, order_seed=seed)
        st = compare.evaluate(y, o, mode)
        assert st["ok"], st


def test_metric_accepts_exact_reference():
    p = make_problem(0)
    for mode in (0, 1, 2):
        o = oracle.swiglu_full(p, mode)
        r, _, _ = compare.reference_values(o, mode)
        assert compare.evaluate(r, o, mode)["max_err"] == 0.0


def _planted(p, kind):
    """A copy of the problem with one plausible implementation mistake."""
    import copy
    q = copy.deepcopy(p)
    if kind == "nibble_order":          # codes read most significant first
        codes = oracle.unpack(q.wg, q.I, q.H, q.bits_g)
        pf = 32 // q.bits_g
        codes = codes.reshape(q.I, -1, pf)[:, :, ::-1].reshape(q.I, q.H)
        q.wg = pack_codes(codes, q.bits_g)
    elif kind == "no_bias":
        q.bg = np.zeros_like(q.bg)
    elif kind == "bias_sign":
        q.bg = q.bg ^ np.uint16(0x8000)
    elif kind == "wrong_group":         # scales of the next group
        q.sg = np.roll(q.sg, 1, axis=1)
    elif kind == "k_tail":              # last 32 inputs dropped
        x = q.x.copy()
        x[:, -32:] = 0
        q.x = x
    elif kind == "swap_gate_up":
        q.wg, q.wu, q.sg, q.su, q.bg, q.bu = q.wu, q.wg, q.su, q.sg, q.bu, q.bg
    elif kind == "transposed_rows":     # output feature rows permuted
        q.wu = q.wu[::-1].copy()
        q.su = q.su[::-1].copy()
        q.bu = q.bu[::-1].copy()
    else:
        raise ValueError(kind)
    return q


@pytest.mark.parametrize("kind", ["nibble_order", "no_bias", "bias_sign", "wrong_group",
                                  "k_tail", "swap_gate_up", "transposed_rows"])
@pytest.mark.parametrize("mode", [0, 1])
def test_metric_catches_planted_mistakes(kind, mode):
    p = make_problem(0)
    o = oracle.swiglu_full(p, mode)
    bad = oracle.swiglu_full(_planted(p, kind), mode)
    r_bad, _, _ = compare.reference_values(bad, mode)
    st = compare.evaluate(r_bad.astype(np.float32), o, mode)
    assert not st["ok"], (kind, st)
    assert st["max_err"] > 50 * compare.TOL[mode], (kind, st)


def test_metric_flags_nonfinite():
    p = make_problem(0)
    o = oracle.swiglu_full(p, 0)
    r, _, _ = compare.reference_values(o, 0)
    r = r.reshape(-1).copy()
    r[5] = np.nan
    assert not compare.evaluate(r, o, 0)["ok"]


def test_bf16_candidates_near_midpoint():
    # 1 + 2^-8 is the midpoint between 1 and 1+2^-7
    v = np.array([1.0 + 2.0**-8 + 2.0**-20, 1.0 + 2.0**-9])
    pv, alt = compare.bf16_candidates(v, np.array([1.0, 1.0]))
    assert pv[0] == 1.0 + 2.0**-7 and alt[0] == 1.0
    assert pv[1] == 1.0 and alt[1] == 1.0      # far from the midpoint
    pv, alt = compare.bf16_candidates(-v, np.array([1.0, 1.0]))
    assert pv[0] == -(1.0 + 2.0**-7) and alt[0] == -1.0


def test_configs_shapes():
    c = CONFIGS
    assert (c[0].M, c[0].H, c[0].I) == (6, 256, 768)
    assert (c[1].M, c[1].H, c[1].I, c[1].calls) == (1, 2048, 5632, 1000)
    assert (c[2].M, c[2].H, c[2].I) == (512, 2048, 8192)
    assert (c[3].M, c[3].H, c[3].I, c[3].x_sigma) == (2048, 4096, 14336, 0.5)
    assert (c[4].bits_g, c[4].gs_g, c[4].bits_u, c[4].gs_u) == (8, 32, 4, 64)
    p = make_problem(0)
    assert p.x.shape == (6, 256) and p.wg.shape == (768, 32) and p.sg.shape == (768, 4)
    s = bf16_bits_to_f32(p.sg)
    assert s.min() >= 0.0049 and s.max() <= 0.0201
    ratio = bf16_bits_to_f32(p.bg) / s
    assert ratio.min() >= -8.8 - 0.1 and ratio.max() <= -7.2 + 0.1


@pytest.mark.parametrize("act,mode", [("bf16", 0), ("bf16", 1), ("bf16", 2), ("f16", 0), ("f16", 1), ("f16", 2)])
def test_metric_allows_the_output_subnormal_rounding_only(act, mode):
    """An output below its type's normal range (silu of a far negative gate)
    is stored as its nearest value of that type; the bar allows that one
    rounding and rejects a quantum more."""
    p = make_custom(1, 256, 64, 4, 64, seed=8, act=act)
    o = oracle.swiglu_full(p, mode)
    o = {k: (v.reshape(-1).copy() if k != "act" else v) for k, v in o.items()}
    q = compare.output_quantum(mode, 1 if act == "f16" else 0)
    # gate far negative: silu(g) u lies between 1 and 2 quanta of the output type
    # (steps of g and u exact in either 16-bit type, so MATCH's rounding keeps them)
    u = -2.125
    g = -16.0
    while abs(g / (1 + np.exp(-g)) * u) > 1.5 * q:
        g -= 1.0 / 64 if act == "f16" else 0.5
    # every element so (a row of one-signed x can do this), else the
    # output's rms would set the floor
    o["g"][:], o["u"][:], o["nu_g"][:], o["nu_u"][:] = g, u, 1e-3, 1e-3
    o["g"][1::2] -= 1.0 / 64 if act == "f16" else 0.5
    r = compare.reference_values(o, mode)[0]
    y = r.copy()
    y[0] = np.round(r[0] / q) * q                   # nearest value of the output type
    assert abs(y[0] - r[0]) > compare.evaluate(r, o, mode)["tol"] * abs(r[0])
    assert compare.evaluate(y, o, mode)["ok"]
    y[0] += q if y[0] >= r[0] else -q               # one quantum further: rejected
    assert not compare.evaluate(y, o, mode)["ok"]
