"""GPU parity of the HIP library (called through its C ABI) against the CPU
oracle, element by element, on seeded synthetic problems: the five workload
configurations (full sizes sampled), a sweep of ragged shapes and
quantization specs through both kernels, the pre-epilogue projections, and
invariants that hold at any size."""
import numpy as np
import pytest
import torch

import oracle
import quantized_swiglu_forward_amd as swq
from gpu_helpers import (skinny_ct, skinny_x, check, device_forward, device_gemm, forced_path, oracle_full, oracle_pairs,
                         sample_pairs, say)
from synth import CONFIGS, bf16_bits_to_f32, make_custom, make_problem, pack_codes, to_bf16_bits

pytestmark = pytest.mark.gpu

GEMV, MFMA = swq.SWQ_PATH_GEMV, swq.SWQ_PATH_MFMA


@pytest.fixture(autouse=True, scope="module")
def _device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    swq.lib()
    yield
    torch.cuda.synchronize()


# ---------------------------------------------------------------- config 0 --

@pytest.mark.parametrize("path", [GEMV, MFMA])
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_config0_full(mode, path):
    p = make_problem(0)
    say("config0", "mode", mode, "path", path)
    y = device_forward(p, mode, path)
    check(y, oracle_full(p, mode), mode, f"c0 mode{mode} path{path}")


def test_config0_default_dispatch():
    p = make_problem(0)
    say("config0 default dispatch")
    expect = swq.swiglu_q_path_for(p.M, p.H, p.I)
    y = device_forward(p, 0, None, expect_path=expect)
    check(y, oracle_full(p, 0), 0, "c0 default")


# ------------------------------------------------------------ shape sweep --

SPECS = [(4, 64, 4, 64), (4, 32, 4, 32), (4, 128, 4, 128), (8, 32, 4, 64), (8, 64, 8, 64),
         (4, 64, 8, 128), (8, 128, 8, 32), (2, 32, 4, 64), (2, 64, 2, 64), (8, 64, 2, 128)]
SHAPES = [(1, 256, 129), (2, 512, 200), (3, 256, 97), (4, 1024, 130), (5, 256, 64), (6, 384, 77),
          (7, 512, 129), (8, 256, 255), (16, 512, 100), (31, 256, 129), (32, 256, 96), (33, 512, 257),
          (63, 256, 65), (64, 128, 64), (65, 512, 300), (127, 256, 129), (128, 256, 128),
          (129, 512, 257), (257, 256, 400)]
SWEEP = []
for i, (M, H, I) in enumerate(SHAPES):
    spec = SPECS[i % len(SPECS)]
    if H % spec[1] or H % spec[3]:
        spec = SPECS[0]
    paths = [GEMV, MFMA] if M <= 32 else [MFMA]
    for path in paths:
        SWEEP.append((M, H, I, spec, i % 3, path))


@pytest.mark.parametrize("M,H,I,spec,mode,path", SWEEP,
                         ids=[f"M{c[0]}-H{c[1]}-I{c[2]}-{c[3][0]}b{c[3][1]}-{c[3][2]}b{c[3][3]}-m{c[4]}-p{c[5]}"
                              for c in SWEEP])
def test_shape_sweep(M, H, I, spec, mode, path):
    bg, gg, bu, gu = spec
    p = make_custom(M, H, I, bg, gg, bu, gu, seed=1000 + M * 7 + I, bias_mode="factor")
    say("sweep", M, H, I, spec, "mode", mode, "path", path)
    y = device_forward(p, mode, path)
    check(y, oracle_full(p, mode), mode, f"sweep M{M} H{H} I{I} {spec} mode{mode} path{path}")


# H not a multiple of 128: the MFMA kernel's last code super-step is partial
# (one to three K-steps of four), on both tile shapes
PARTIAL = [(70, 96, 130, (4, 32, 4, 32)), (300, 160, 200, (8, 32, 4, 32)), (129, 2080, 257, (2, 32, 8, 32)),
           (600, 2080, 384, (4, 32, 4, 32))]


@pytest.mark.parametrize("tiles", ["0", "1"], ids=["256x128", "128x128"])
@pytest.mark.parametrize("M,H,I,spec", PARTIAL, ids=[f"M{m}-H{h}-I{i}" for m, h, i, _ in PARTIAL])
def test_partial_super_step(M, H, I, spec, tiles):
    import os
    p = make_custom(M, H, I, *spec, seed=M + H + I)
    mode = (M + H) % 3
    say("partial super-step", M, H, I, spec, "tiles", tiles, "mode", mode)
    old = os.environ.get("SWIGLU_Q_MFMA_CFG")
    os.environ["SWIGLU_Q_MFMA_CFG"] = tiles
    try:
        y = device_forward(p, mode, MFMA)
    finally:
        if old is None:
            os.environ.pop("SWIGLU_Q_MFMA_CFG", None)
        else:
            os.environ["SWIGLU_Q_MFMA_CFG"] = old
    check(y, oracle_full(p, mode), mode, f"partial M{M} H{H} tiles{tiles}")


@pytest.mark.parametrize("case", range(12))
def test_random_specs_and_magnitudes(case):
    """Seeded random problems on both paths: any gate/up code widths and
    group sizes, ragged I, x scaled from 2^-10 to 2^10 and scales anywhere in
    the documented exact range [2^-17, 2^8), every precision mode."""
    rng = np.random.default_rng(500 + case)
    bits_g, bits_u = (int(b) for b in rng.choice([2, 4, 8], 2))
    gs_g, gs_u = (int(g) for g in rng.choice([32, 64, 128], 2))
    M = int(rng.choice([1, 3, 9, 40, 200]))
    H = int(rng.choice([256, 512, 1024]))
    I = int(rng.integers(33, 300))
    s_lo = float(2.0 ** rng.uniform(-17, 6))
    mode = case % 3
    p = make_custom(M, H, I, bits_g, gs_g, bits_u, gs_u, seed=700 + case,
                    x_sigma=float(2.0 ** rng.uniform(-10, 10)), s_lo=s_lo, s_hi=s_lo * 4)
    path = GEMV if M <= 16 and case % 2 == 0 else MFMA
    say("random", M, H, I, (bits_g, gs_g, bits_u, gs_u), "s_lo", s_lo, "mode", mode, "path", path)
    y = device_forward(p, mode, path)
    check(y, oracle_full(p, mode), mode, f"random case {case}")


@pytest.mark.parametrize("case", range(16))
def test_random_few_row_forms(case):
    """Seeded random problems on the matrix-vector path for 2 <= M <= 128:
    any code widths and group sizes, H from 64 to 2560 (ragged in chunk
    quads), ragged I, both activation types, every mode, with the library's
    choice or a forced column-tile count, x source and quads per wave."""
    rng = np.random.default_rng(900 + case)
    narrow = case % 3 != 0
    if narrow:
        bits_g = bits_u = int(rng.choice([2, 4]))
    else:
        bits_g, bits_u = (int(b) for b in rng.choice([2, 4, 8], 2))
    gs_g, gs_u = (int(g) for g in rng.choice([32, 64, 128], 2))
    step = max(gs_g, gs_u)
    M = int(rng.choice([2, 5, 8, 11, 16, 17, 25, 32, 33, 47, 64, 65, 100, 128]))
    H = step * int(rng.integers(1, 2560 // step + 1))
    I = int(rng.integers(1, 700))
    act = "f16" if case % 4 == 1 else "bf16"
    mode = case % 3
    ct = [None, 1, 2][case % 3]
    quads = 1 if case % 5 == 2 else None
    source = "prep" if case % 7 == 3 else None
    p = make_custom(M, H, I, bits_g, gs_g, bits_u, gs_u, seed=1000 + case, act=act)
    say("random few-row", M, H, I, (bits_g, gs_g, bits_u, gs_u), act, "mode", mode, "ct", ct, "quads", quads,
        "x source", source)
    with skinny_ct(ct, quads), skinny_x(source):
        y = device_forward(p, mode, GEMV)
    check(y, oracle_full(p, mode), mode, f"random few-row case {case}")


# ------------------------------------------- scale and bias magnitudes --

# Scales and biases anywhere in bf16's range: each weight row's scales and
# constants get their own power of two before they become binary16 operands,
# so every kernel stays finite and exact (up to float32 accumulation) for
# tiny and huge scales, scales that differ by many binades between the groups
# of one row, and large biases.
RANGE_LAWS = [
    ("s2m24", (4, 64, 4, 64), ("pow", -24), "factor"),
    ("s2m20", (4, 64, 4, 64), ("pow", -20), "factor"),
    ("s2p10", (4, 64, 4, 64), ("pow", 10), "factor"),
    ("s2p14", (4, 64, 4, 64), ("pow", 14), "factor"),
    ("8bit-s2p10", (8, 32, 8, 64), ("pow", 10), "half"),
    ("mixed-groups", (4, 64, 8, 32), ("mixed", -20, 14), "factor"),
    ("bias1e5", (4, 64, 4, 64), ("pow", -7), ("uniform", 1e5)),
    ("8bit-mixed-bias1e5", (8, 32, 2, 64), ("mixed", -20, 10), ("uniform", 1e5)),
    ("x2p60-s2m60", (4, 64, 8, 32), ("pow", -60), "factor", 60),
    ("x2m50-s2p20", (4, 32, 4, 64), ("mixed", 10, 20), "factor", -50),
]
# (M, H, I, path): the M = 1 kernel, its several-row form, the few-row kernel
# with x' built in the block and from the prep kernel (one and two row tiles),
# and the MFMA kernel
RANGE_SHAPES = [(1, 1024, 130, GEMV), (3, 2048, 70, GEMV), (6, 512, 97, GEMV), (9, 2048, 66, GEMV),
                (20, 1024, 50, GEMV), (70, 512, 130, MFMA)]
RANGE_CASES = [(law, shape) for law in RANGE_LAWS for shape in RANGE_SHAPES]


def _range_problem(M, H, I, spec, s_law, b_law, seed, x_exp=0):
    bits_g, gs_g, bits_u, gs_u = spec
    p = make_custom(M, H, I, bits_g, gs_g, bits_u, gs_u, seed=seed, x_sigma=float(2.0 ** x_exp))
    rng = np.random.default_rng(seed)
    for tag, bits, gs in (("g", bits_g, gs_g), ("u", bits_u, gs_u)):
        shape = (I, H // gs)
        if s_law[0] == "pow":
            s = np.float32(2.0 ** s_law[1]) * rng.uniform(1.0, 2.0, shape).astype(np.float32)
        else:
            s = np.exp2(rng.uniform(s_law[1], s_law[2], shape)).astype(np.float32)
        s_bits = to_bf16_bits(s)
        sv = bf16_bits_to_f32(s_bits)
        if b_law == "factor":
            b = np.float32(-(1 << (bits - 1))) * sv * rng.uniform(0.9, 1.1, shape).astype(np.float32)
        elif b_law == "half":
            b = np.float32(-(1 << (bits - 1))) * sv
        else:
            b = rng.uniform(-b_law[1], b_law[1], shape).astype(np.float32)
        setattr(p, "s" + tag, s_bits)
        setattr(p, "b" + tag, to_bf16_bits(b.astype(np.float32)))
    return p


@pytest.mark.parametrize("law,shape", RANGE_CASES,
                         ids=[f"{l[0]}-M{sh[0]}-H{sh[1]}-p{sh[3]}" for l, sh in RANGE_CASES])
def test_scale_and_bias_range(law, shape):
    name, spec, s_law, b_law = law[:4]
    x_exp = law[4] if len(law) > 4 else 0
    M, H, I, path = shape
    mode = (len(name) + M) % 3
    p = _range_problem(M, H, I, spec, s_law, b_law, seed=M * 131 + H + len(name), x_exp=x_exp)
    say("range", name, M, H, I, spec, "mode", mode, "path", path)
    o = oracle_full(p, mode)
    g, u = device_gemm(p, path)
    assert np.all(np.isfinite(g)) and np.all(np.isfinite(u)), name
    eg = np.max(np.abs(g - o["g"]) / o["nu_g"])
    eu = np.max(np.abs(u - o["u"]) / o["nu_u"])
    print(f"  {name}: max |dg|/nu_g={eg:.3g} |du|/nu_u={eu:.3g}")
    assert eg <= 1e-5 and eu <= 1e-5, (eg, eu)
    y = device_forward(p, mode, path)
    check(y, o, mode, f"range {name} M{M} H{H} path{path}")


# ------------------------------------------------------- decode (M = 1) --

# every branch of the M = 1 kernel: a whole wave per column with one to four
# chunks per lane (H = 2048, 4096, 6144, 8192), with idle lanes (H = 3072,
# 5632, 7168), fewer lanes per column (H = 1024, 512), one and two columns
# per wave (I below and above 4096), all three code widths (2, 4, 8) and all group sizes on
# each side, ragged I
DECODE_CASES = [
    (2048, 5633, (4, 64, 4, 64)), (2048, 301, (8, 32, 4, 64)), (2048, 257, (4, 128, 8, 128)),
    (2048, 130, (8, 64, 8, 32)), (4096, 515, (4, 64, 4, 64)), (4096, 129, (8, 128, 4, 32)),
    (3072, 200, (4, 64, 8, 64)), (1024, 333, (4, 32, 4, 128)), (512, 97, (8, 64, 4, 64)),
    (6144, 300, (4, 64, 4, 64)), (5632, 257, (8, 32, 4, 64)), (8192, 130, (4, 128, 8, 64)),
    (7168, 77, (8, 64, 8, 32)), (8192, 4100, (4, 64, 4, 64)),
    (2048, 300, (2, 64, 2, 64)), (4096, 129, (2, 32, 8, 64)), (5632, 90, (4, 128, 2, 32)),
]


@pytest.mark.parametrize("H,I,spec", DECODE_CASES, ids=[f"H{h}-I{i}-{s[0]}b{s[1]}-{s[2]}b{s[3]}" for h, i, s in DECODE_CASES])
@pytest.mark.parametrize("mode", [0, 1])
def test_decode_branches(H, I, spec, mode):
    p = make_custom(1, H, I, *spec, seed=H + I)
    say("decode", H, I, spec, "mode", mode)
    y = device_forward(p, mode, GEMV)
    check(y, oracle_full(p, mode), mode, f"decode H{H} I{I} {spec} mode{mode}")


# ------------------------------------------- decode, a few rows (M <= 4) --

# the several-row form of the matrix-vector kernel (2 <= M <= 4,
# 2048 <= H <= 4096): one and two chunks per lane (H = 2048, 4096), idle lanes
# (H = 2560, 3072, 3584), one and two columns per wave (I below and above
# 4096), every code width on each side, ragged I, every precision mode
ROWS_CASES = [
    (2, 2048, 5633, (4, 64, 4, 64)), (3, 2048, 301, (8, 32, 4, 64)), (4, 2048, 130, (2, 64, 8, 32)),
    (2, 4096, 515, (4, 64, 4, 64)), (4, 4096, 129, (8, 128, 2, 32)), (3, 3072, 200, (4, 64, 8, 64)),
    (4, 2560, 333, (4, 32, 4, 128)), (2, 3584, 97, (8, 64, 4, 64)), (4, 2048, 4100, (2, 32, 2, 64)),
    (3, 4096, 4097, (4, 64, 4, 64)), (2, 3072, 4200, (8, 32, 4, 64)),
]


@pytest.mark.parametrize("M,H,I,spec", ROWS_CASES,
                         ids=[f"M{m}-H{h}-I{i}-{s[0]}b{s[1]}-{s[2]}b{s[3]}" for m, h, i, s in ROWS_CASES])
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_decode_rows(M, H, I, spec, mode):
    p = make_custom(M, H, I, *spec, seed=M * 1000 + H + I)
    say("decode rows", M, H, I, spec, "mode", mode)
    y = device_forward(p, mode, GEMV)
    check(y, oracle_full(p, mode), mode, f"decode rows M{M} H{H} I{I} {spec} mode{mode}")


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("M,H,I", [(4, 2048, 300), (3, 3072, 300), (2, 4096, 300), (4, 2048, 4100), (3, 3584, 4500)])
def test_decode_rows_match_single_row_calls(M, H, I):
    """Each row of a several-row call takes the single-row call's arithmetic
    in the same order (the same columns per wave, chunks per lane and
    reduction), so the results agree bit for bit."""
    p = make_custom(M, H, I, 4, 64, 8, 32, seed=H + I)
    dev = swq.to_device(p)
    say("rows vs single-row calls", M, H, I)
    with forced_path(GEMV, M):
        for mode in (0, 1):
            whole = swq.forward(*dev, p.bits_g, p.gs_g, p.bits_u, p.gs_u, mode=mode)
            for m in range(M):
                one = swq.forward(dev[0][m:m + 1].contiguous(), *dev[1:], p.bits_g, p.gs_g, p.bits_u, p.gs_u,
                                  mode=mode)
                torch.cuda.synchronize()
                assert torch.equal(_bits(whole[m:m + 1]), _bits(one)), (M, H, I, mode, m)


# ------------------------------------------------------- full-size configs --

@pytest.mark.parametrize("mode", [0, 1])
def test_config1_decode_full(mode):
    p = make_problem(1)
    say("config1 decode full", "mode", mode)
    y = device_forward(p, mode, None, expect_path=swq.swiglu_q_path_for(1, p.H, p.I))
    check(y, oracle_full(p, mode), mode, f"c1 mode{mode}")


def test_config1_fresh_inputs():
    """Three of the 1000 fresh decode inputs, on one resident weight set."""
    p = make_problem(1)
    dev = list(swq.to_device(p))
    for call in (0, 499, 999):
        q = make_problem(1, with_calls=False)
        q.x = p.xs[call:call + 1].copy()
        dev[0] = swq.to_device(q)[0]
        say("config1 fresh x call", call)
        y = device_forward(q, 0, None, dev=tuple(dev))
        check(y, oracle_full(q, 0), 0, f"c1 call {call}")


def tile_cover_pairs(M, I, seed, tile=128):
    """For every tile x tile block of an [M, I] output, one sample in each of
    its rows and each of its columns (a random permutation within the block).
    Every output tile of either MFMA tile shape (256 x 128 or 128 x 128, and
    the columns of a split launch, which start on a multiple of 128) then has
    a sample in every row -- every fragment and lane of every wave -- and in
    every column -- every wave, 32-column slice and accumulator entry."""
    rng = np.random.default_rng(seed)
    ms, ns = [], []
    for m0 in range(0, M, tile):
        rows = min(tile, M - m0)
        for n0 in range(0, I, tile):
            cols = min(tile, I - n0)
            k = max(rows, cols)
            ms.append(m0 + np.arange(k) % rows)
            ns.append(n0 + rng.permutation(k) % cols)
    return np.concatenate(ms).astype(np.int64), np.concatenate(ns).astype(np.int64)


_FULL_ORACLE = {}


def _full_size_oracle(cfg):
    """Configuration 2 in full; 3 and 4 on tile-covering samples.  The
    oracle's gate, up and scales do not depend on the precision mode, so one
    evaluation serves every mode."""
    if cfg not in _FULL_ORACLE:
        p = make_problem(cfg)
        c = CONFIGS[cfg]
        if cfg == 2:
            ms = ns = None
        else:
            ms, ns = tile_cover_pairs(c.M, c.I, seed=cfg)
        o = oracle.swiglu_pairs(p, 1, ms, ns, want=("g", "u", "nu_g", "nu_u"))
        _FULL_ORACLE.clear()                            # one configuration held at a time
        _FULL_ORACLE[cfg] = (p, ms, ns, o)
    return _FULL_ORACLE[cfg]


@pytest.mark.parametrize("cfg,mode", [(2, 0), (2, 1), (2, 2), (3, 0), (3, 1), (4, 0), (4, 1)])
def test_full_size(cfg, mode):
    """The prefill configurations at full size in the launch configuration
    the benchmark times: every output of configuration 2, and at least one
    output per row and per column of every 128 x 128 block of 3 and 4."""
    p, ms, ns, o = _full_size_oracle(cfg)
    say(f"config{cfg} full size", "mode", mode, "samples", "all" if ms is None else ms.size)
    y = device_forward(p, mode, None, expect_path=MFMA)
    assert np.all(np.isfinite(y))
    got = y.reshape(-1) if ms is None else y[ms, ns]
    check(got, o, mode, f"c{cfg} mode{mode} " + ("all outputs" if ms is None else f"{ms.size} tile-covering samples"))


# large extents: H at 64 K inputs on every kernel (x' and the weight rows
# addressed with 32-bit offsets far from 0), M beyond 65,536 rows, I beyond
# 100 K columns, sampled outputs against the oracle
LARGE = [(1, 65536, 100, (4, 64, 4, 64), GEMV), (4, 65536, 70, (8, 32, 4, 128), GEMV),
         (64, 65536, 200, (4, 64, 8, 64), MFMA), (70000, 256, 96, (4, 64, 4, 64), MFMA),
         (3, 1024, 120000, (4, 32, 4, 64), GEMV), (2, 4096, 40000, (4, 64, 4, 64), GEMV)]


@pytest.mark.parametrize("M,H,I,spec,path", LARGE, ids=[f"M{c[0]}-H{c[1]}-I{c[2]}" for c in LARGE])
def test_large_extents_sampled(M, H, I, spec, path):
    p = make_custom(M, H, I, *spec, seed=M + I)
    mode = (M + I) % 3
    say("large extents", M, H, I, spec, "mode", mode, "path", path)
    y = device_forward(p, mode, path)
    ms, ns = sample_pairs(M, I, 600, seed=H)
    o = oracle_pairs(p, mode, ms, ns)
    check(y[ms, ns], o, mode, f"large M{M} H{H} I{I}")
    assert np.all(np.isfinite(y))


# -------------------------------------------------- pre-epilogue gate / up --

@pytest.mark.parametrize("path", [GEMV, MFMA])
@pytest.mark.parametrize("spec", [(4, 64, 4, 64), (8, 32, 4, 64), (4, 128, 8, 64)])
def test_debug_gemm_matches_oracle(spec, path):
    M = 5 if path == GEMV else 70
    p = make_custom(M, 1024, 193, *spec, seed=31)
    say("debug gemm", spec, "path", path)
    g, u = device_gemm(p, path)
    o = oracle_full(p, 1)
    eg = np.max(np.abs(g - o["g"]) / o["nu_g"])
    eu = np.max(np.abs(u - o["u"]) / o["nu_u"])
    print(f"  max |dg|/nu_g={eg:.3g} |du|/nu_u={eu:.3g}")
    assert eg <= 1e-5 and eu <= 1e-5


@pytest.mark.parametrize("path", [GEMV, MFMA])
def test_integer_special_case_is_exact(path):
    """s = 1, b in {0, -8}, small-integer x: gate and up are integers below
    2^24 and must come out bit-exact."""
    rng = np.random.default_rng(5)
    M, H, I = (3, 512, 70) if path == GEMV else (40, 512, 70)
    p = make_custom(M, H, I, 8, 32, 4, 64, seed=2)
    xi = rng.integers(-7, 8, size=(M, H))
    p.x = to_bf16_bits(xi.astype(np.float32))
    cg = rng.integers(0, 256, size=(I, H), dtype=np.uint8)
    cu = rng.integers(0, 16, size=(I, H), dtype=np.uint8)
    p.wg, p.wu = pack_codes(cg, 8), pack_codes(cu, 4)
    p.sg = to_bf16_bits(np.ones((I, H // 32), np.float32))
    p.bg = to_bf16_bits(np.zeros((I, H // 32), np.float32))
    p.su = to_bf16_bits(np.ones((I, H // 64), np.float32))
    p.bu = to_bf16_bits(np.full((I, H // 64), -8.0, np.float32))
    say("integer exact", "path", path)
    g, u = device_gemm(p, path)
    ref_g = xi @ cg.astype(np.int64).T
    ref_u = xi @ (cu.astype(np.int64) - 8).T
    assert np.array_equal(g, ref_g.astype(np.float64))
    assert np.array_equal(u, ref_u.astype(np.float64))


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8, 17, 24, 32])
def test_gemv_and_mfma_agree(M):
    p = make_custom(M, 2048, 300, 4, 64, seed=M)
    say("gemv vs mfma", M)
    yg = device_forward(p, 1, GEMV)
    ym = device_forward(p, 1, MFMA)
    o = oracle_full(p, 1)
    check(yg, o, 1, f"gemv M{M}")
    check(ym, o, 1, f"mfma M{M}")


# the few-row kernel with one and two tiles of 16 rows (M up to 32), every x
# source the shape allows (converted by each wave, built in the block's LDS
# for M*H <= 8192, staged by the prep kernel), all three code widths, and
# M <= 4 and M = 1 past the matrix-vector kernel's H limits
FEW_ROW = [(6, 1024, 130, (4, 64, 8, 32)), (2, 8192, 97, (4, 64, 4, 64)), (8, 1024, 257, (8, 64, 4, 128)),
           (5, 2048, 96, (4, 32, 4, 64)), (9, 2048, 300, (4, 64, 4, 64)), (16, 2048, 129, (8, 32, 8, 64)),
           (12, 4096, 64, (4, 128, 4, 64)), (16, 512, 100, (4, 64, 8, 64)), (1, 8192, 200, (4, 64, 4, 64)),
           (1, 16384, 33, (8, 64, 4, 32)), (1, 32768, 40, (4, 64, 4, 64)), (5, 1024, 77, (2, 64, 4, 64)),
           (12, 2048, 96, (2, 128, 2, 32)), (3, 6144, 50, (8, 32, 2, 64)), (4, 5120, 70, (4, 64, 4, 64)),
           (17, 2048, 130, (4, 64, 8, 32)), (24, 256, 97, (4, 64, 4, 64)), (32, 256, 200, (8, 32, 2, 64)),
           (32, 4096, 65, (4, 128, 4, 64)), (20, 1024, 77, (2, 64, 8, 128)), (29, 448, 33, (4, 64, 4, 64))]


@pytest.mark.parametrize("M,H,I,spec", FEW_ROW, ids=[f"M{m}-H{h}-I{i}" for m, h, i, _ in FEW_ROW])
def test_few_row_kernel_x_staging(M, H, I, spec):
    mode = (M + H // 1024) % 3
    p = make_custom(M, H, I, *spec, seed=M * 31 + I)
    o = oracle_full(p, mode)
    dev = swq.to_device(p)
    for source in [None, "prep"] + (["stage"] if M * H <= 8192 else []):
        say("few-row", M, H, I, spec, "mode", mode, "x source", source or "default")
        with skinny_x(source):
            y = device_forward(p, mode, GEMV, dev=dev)
        check(y, o, mode, f"few-row M{M} H{H} I{I} x source {source}")


# x converted by each wave of the few-row kernel with its own row exponents:
# rows whose magnitudes differ by row and by 256-input slice (the waves of a
# block see different slices), a row that is zero over half of H (whole waves
# see only zeros), bf16 subnormals, ragged H, pairs past the last in the
# waves' x loads (M * chunks not a multiple of 16); one and two chunk quads
# per wave, one and two row tiles, narrow, mixed and 8-bit codes
SELF_CASES = [(8, 2048, (4, 64, 4, 64)), (13, 2048, (8, 32, 8, 64)), (8, 4096, (4, 128, 4, 128)),
              (16, 2048, (4, 64, 8, 32)), (5, 1056, (2, 32, 2, 32)), (16, 1024, (4, 32, 4, 64)),
              (2, 1024, (4, 64, 4, 64)), (3, 1184, (8, 32, 4, 32)), (24, 2048, (4, 64, 4, 64)),
              (32, 1056, (2, 32, 2, 32)), (17, 2048, (4, 128, 4, 128))]


@pytest.mark.parametrize("M,H,spec", SELF_CASES, ids=[f"M{m}-H{h}" for m, h, _ in SELF_CASES])
def test_few_row_wave_exponents(M, H, spec):
    from synth import bf16_bits_to_f32, to_bf16_bits
    assert swq.swiglu_q_staging_bytes(M, H, 97, *spec) == 0, "x converted in the kernel"
    p = make_custom(M, H, 97, *spec, seed=M * 7 + H)
    rng = np.random.default_rng(M + H)
    x = bf16_bits_to_f32(p.x).astype(np.float64)
    x *= np.exp2(rng.integers(-20, 21, M))[:, None]
    x *= np.repeat(np.exp2(rng.integers(-20, 21, (H + 255) // 256)), 256)[None, :H]
    x[M // 2, : H // 2] = 0.0
    x[-1, ::7] = rng.choice([1e-39, -3e-40, 5e-41, -7e-42], x[-1, ::7].size)
    p.x = to_bf16_bits(x.astype(np.float32))
    say("wave exponents", M, H, spec)
    y = device_forward(p, 1, GEMV)
    check(y, oracle_full(p, 1), 1, f"wave exponents M{M} H{H}")


# two column tiles per block of the few-row kernel (x converted by the waves,
# one chunk quad per wave): the decode width (the default picks two tiles
# there), ragged widths whose last block has a partial or an empty second
# tile, 2- and 4-bit codes, gs 32 to 128, both activation types, one and
# two row tiles (ragged H too).  Each
# column's arithmetic is that of one tile per block with one quad per wave,
# so the two agree bit for bit; every form passes against the oracle on
# every output.
CT2_CASES = [(8, 2048, 5632, (4, 64, 4, 64), "bf16"), (5, 1024, 1000, (4, 64, 4, 64), "bf16"),
             (16, 2048, 56, (2, 32, 2, 32), "bf16"), (13, 512, 40, (4, 128, 4, 128), "bf16"),
             (9, 1536, 300, (4, 32, 4, 32), "bf16"), (8, 2048, 33, (4, 64, 4, 64), "f16"),
             (16, 2048, 600, (2, 64, 2, 64), "f16"), (6, 2048, 5632, (4, 64, 4, 64), "f16"),
             # two row tiles (16 < M <= 32)
             (24, 2048, 5632, (4, 64, 4, 64), "bf16"), (17, 1024, 1000, (4, 64, 4, 64), "bf16"),
             (32, 2048, 56, (2, 32, 2, 32), "f16"), (20, 512, 600, (4, 128, 4, 128), "bf16"),
             (29, 1504, 130, (4, 32, 4, 32), "f16")]


@pytest.mark.parametrize("M,H,I,spec,act", CT2_CASES, ids=[f"M{m}-H{h}-I{i}-{a}" for m, h, i, _, a in CT2_CASES])
def test_few_row_two_column_tiles(M, H, I, spec, act):
    mode = (M + I) % 3
    p = make_custom(M, H, I, *spec, seed=M * 5 + I, act=act)
    assert swq.swiglu_q_staging_bytes(M, H, I, *spec) == 0, "x converted by the waves"
    o = oracle_full(p, mode)
    dev = swq.to_device(p)
    ys = {}
    for key, ct, quads in (("one tile", 1, None), ("one tile, one quad", 1, 1), ("two tiles", 2, None),
                           ("default", None, None)):
        say("few-row column tiles", M, H, I, spec, act, "mode", mode, key)
        with skinny_ct(ct, quads):
            ys[key] = device_forward(p, mode, GEMV, dev=dev)
        check(ys[key], o, mode, f"few-row M{M} H{H} I{I} {act} {key}")
    assert np.array_equal(ys["one tile, one quad"], ys["two tiles"]), "one and two column tiles differ"
    tiles = (I + 15) // 16
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert np.array_equal(ys["default"], ys["two tiles" if cus < tiles <= 2 * cus else "one tile"])


# row groups of 32 (33 <= M <= 128 on the matrix-vector path): x converted by
# the waves of each group or staged by the prep kernel for every group (8-bit
# or mixed codes, H past one pass, or forced), 2 to 4 groups, a last group of
# one row, ragged widths and ragged H (a partial last chunk quad), both
# activation types; every output against the oracle (sampled at the decode
# width)
ROW_GROUP_CASES = [(33, 2048, 300, (4, 64, 4, 64), "bf16"), (48, 1024, 1000, (4, 64, 4, 64), "bf16"),
                   (64, 2048, 5632, (4, 64, 4, 64), "bf16"), (96, 512, 200, (2, 32, 2, 32), "f16"),
                   (128, 2048, 130, (4, 128, 4, 128), "bf16"), (40, 2048, 257, (8, 32, 4, 64), "bf16"),
                   (70, 4096, 100, (4, 64, 4, 64), "bf16"), (100, 1024, 77, (2, 64, 8, 128), "f16"),
                   (65, 256, 97, (4, 64, 4, 64), "bf16"), (40, 1056, 77, (2, 32, 2, 32), "bf16"),
                   (72, 1184, 50, (8, 32, 4, 32), "f16"), (120, 1504, 33, (4, 32, 4, 32), "bf16")]


@pytest.mark.parametrize("M,H,I,spec,act", ROW_GROUP_CASES, ids=[f"M{m}-H{h}-I{i}-{a}" for m, h, i, _, a in ROW_GROUP_CASES])
def test_few_row_row_groups(M, H, I, spec, act):
    mode = (M + I) % 3
    p = make_custom(M, H, I, *spec, seed=M * 3 + I, act=act)
    dev = swq.to_device(p)
    if M * I > 100000:
        rng = np.random.default_rng(M)
        ms = np.concatenate([np.arange(M), rng.integers(0, M, 3000)])
        ns = np.concatenate([rng.integers(0, I, M), rng.integers(0, I, 3000)])
        ref = oracle_pairs(p, mode, ms, ns)
    else:
        ms = ns = None
        ref = oracle_full(p, mode)
    for source in (None, "prep"):
        say("row groups", M, H, I, spec, act, "mode", mode, "x source", source or "default")
        with skinny_x(source):
            y = device_forward(p, mode, GEMV, dev=dev)
        check(y if ms is None else y[ms, ns], ref, mode, f"row groups M{M} H{H} I{I} {act} x source {source}")


# ------------------------------------------------- tile shapes and splits --

def test_tile_shapes_and_column_split_agree_bitwise():
    """M=512, I=38400 gives 600 tiles of 256 x 128: two whole rounds on 256
    CUs, so the columns past them run as 128 x 128 tiles in a second launch.
    Every output accumulates the same products in the same order whatever
    the tile shape, so the split launch, the single 256 x 128 launch and the
    all-128 x 128 launch agree bit for bit; sampled outputs on both sides of
    the split column are checked against the oracle."""
    import os
    p = make_custom(512, 256, 38400, 4, 64, 4, 64, seed=41)
    dev = swq.to_device(p)
    outs = {}
    for name, env in (("split", {}), ("single", {"SWIGLU_Q_MFMA_SPLIT": "0"}), ("small", {"SWIGLU_Q_MFMA_CFG": "1"})):
        say("tile shapes", name)
        saved = {k: os.environ.get(k) for k in ("SWIGLU_Q_MFMA_SPLIT", "SWIGLU_Q_MFMA_CFG")}
        try:
            for k in saved:
                os.environ.pop(k, None)
            os.environ.update(env)
            outs[name] = device_forward(p, 1, MFMA, dev=dev)
        finally:
            for k, v in saved.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v
    assert np.array_equal(outs["split"], outs["single"])
    assert np.array_equal(outs["split"], outs["small"])
    rng = np.random.default_rng(3)
    ns = np.concatenate([np.arange(32768 - 64, 32768 + 64), rng.integers(0, 38400, 200)])
    ms = rng.integers(0, 512, ns.size)
    o = oracle_pairs(p, 1, ms, ns)
    check(outs["split"][ms, ns], o, 1, "split boundary sampled")


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_output_alignment_paths_agree_bitwise(mode):
    """The matrix-matrix epilogue writes four consecutive features per store
    when the output rows allow it (I a multiple of 4, output 16-byte
    aligned) and one element per store otherwise.  An output view that
    starts one element into a larger buffer takes the element path; both
    paths must write the same bits, and match the oracle."""
    M, H, I = 300, 256, 200
    p = make_custom(M, H, I, 4, 64, 8, 32, seed=77)
    dev = swq.to_device(p)
    dt = torch.float32 if mode == 1 else torch.bfloat16
    say("alignment", mode)
    with forced_path(MFMA, M):
        a = swq.forward(*dev, p.bits_g, p.gs_g, p.bits_u, p.gs_u, mode=mode)
        big = torch.full((M * I + 8,), float("nan"), dtype=dt, device="cuda")
        b = big[1:1 + M * I].view(M, I)
        assert b.data_ptr() % 16 != 0
        swq.forward(*dev, p.bits_g, p.gs_g, p.bits_u, p.gs_u, mode=mode, out=b)
    torch.cuda.synchronize()
    ya = a.float().cpu().numpy().astype(np.float64)
    yb = b.float().cpu().numpy().astype(np.float64)
    assert np.array_equal(ya, yb)
    assert torch.isnan(big[0]).item() and torch.isnan(big[1 + M * I:]).all().item()
    check(ya, oracle_full(p, mode), mode, f"alignment mode{mode}")


# -------------------------------------------------------------- invariants --

@pytest.mark.parametrize("path", [GEMV, MFMA])
def test_bitwise_repeatable(path):
    p = make_custom(8 if path == GEMV else 300, 1024, 500, 4, 64, seed=12)
    dev = swq.to_device(p)
    say("repeatability", path)
    a = device_forward(p, 0, path, dev=dev)
    b = device_forward(p, 0, path, dev=dev)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("path", [GEMV, MFMA])
def test_row_and_column_permutation(path):
    M = 6 if path == GEMV else 200
    p = make_custom(M, 512, 160, 8, 32, 4, 64, seed=13)
    say("permutation", path)
    y = device_forward(p, 1, path)
    rng = np.random.default_rng(0)
    pr = rng.permutation(M)
    pc = rng.permutation(160)
    q = make_custom(M, 512, 160, 8, 32, 4, 64, seed=13)
    q.x = p.x[pr].copy()
    for k in ("wg", "sg", "bg", "wu", "su", "bu"):
        setattr(q, k, getattr(p, k)[pc].copy())
    yq = device_forward(q, 1, path)
    assert np.array_equal(yq, y[pr][:, pc])


@pytest.mark.parametrize("path", [GEMV, MFMA])
def test_power_of_two_scaling_of_x(path):
    M = 4 if path == GEMV else 100
    p = make_custom(M, 1024, 96, 4, 64, seed=14)
    say("x scaling", path)
    g1, u1 = device_gemm(p, path)
    q = make_custom(M, 1024, 96, 4, 64, seed=14)
    q.x = to_bf16_bits(bf16_bits_to_f32(p.x) * np.float32(8.0))
    g8, u8 = device_gemm(q, path)
    assert np.array_equal(g8, 8.0 * g1) and np.array_equal(u8, 8.0 * u1)


@pytest.mark.parametrize("path", [GEMV, MFMA])
def test_zero_gate_weights(path):
    """Constant codes c per group with b = -s*c: every gate weight is zero, so
    hidden is zero up to float32 rounding of the terms that cancel."""
    M = 3 if path == GEMV else 64
    p = make_custom(M, 512, 90, 4, 64, seed=15)
    rng = np.random.default_rng(15)
    c = rng.choice(np.array([1, 2, 4, 8]), size=(90, 512 // 64))
    p.wg = pack_codes(np.repeat(c, 64, axis=1).astype(np.uint8), 4)
    s = bf16_bits_to_f32(p.sg)
    p.bg = to_bf16_bits((-s * c).astype(np.float32))
    say("zero gate", path)
    g, _ = device_gemm(p, path)
    scale = np.abs(bf16_bits_to_f32(p.x)).astype(np.float64).sum(axis=1, keepdims=True) * float(s.max()) * 8
    assert np.all(np.abs(g) <= 2.0 ** -20 * scale)
    y = device_forward(p, 1, path)
    o = oracle_full(p, 1)
    assert np.all(o["h"] == 0.0)
    assert np.all(np.abs(y) <= 2.0 ** -18 * scale * np.abs(o["u"]).max())


def test_m_zero_launches_nothing():
    p = make_custom(1, 256, 64, 4, 64, seed=1)
    dev = swq.to_device(p)
    out = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    before = [swq.swiglu_q_call_count(k) for k in (0, 1)]
    rc = swq.swiglu_q_forward(dev[0], *dev[1:], 0, 256, 64, 4, 64, 4, 64, 0, out.data_ptr() or 256, None)
    assert rc == swq.SWQ_OK
    assert [swq.swiglu_q_call_count(k) for k in (0, 1)] == before


# ---------------------------------------------------------------- HIP graphs --

@pytest.mark.parametrize("M,H,I,spec", [(1, 2048, 600, (4, 64, 4, 64)), (3, 2048, 600, (4, 64, 4, 64)),
                                        (6, 256, 300, (8, 32, 4, 64)), (12, 2048, 200, (4, 64, 4, 64)),
                                        (24, 1024, 300, (4, 64, 4, 64)), (20, 2048, 200, (8, 32, 4, 64)),
                                        (48, 2048, 600, (4, 64, 4, 64)), (40, 2048, 300, (8, 32, 4, 64)),
                                        (300, 512, 384, (4, 64, 8, 32))],
                         ids=["decode", "decode-rows", "few-row-in-block", "few-row-waves", "few-row-two-row-tiles",
                              "few-row-prep", "row-groups", "row-groups-prep", "mfma"])
def test_graph_replays_match_eager(M, H, I, spec):
    """The forward recorded into a HIP graph (after an eager call, so the
    workspace exists) and replayed several times, with other eager work and
    synchronisations between the replays, writes the eager result every
    time: the kernels and the workspace they share need no per-call clearing."""
    p = make_custom(M, H, I, *spec, seed=M + I)
    dev = swq.to_device(p)
    say("graph", M, H, I, spec)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):                   # the workspace belongs to (device, stream)
        eager = swq.forward(*dev, p.bits_g, p.gs_g, p.bits_u, p.gs_u, mode=0, stream=stream)
    torch.cuda.synchronize()
    ref = eager.clone()
    out = torch.empty_like(eager)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        swq.forward(*dev, p.bits_g, p.gs_g, p.bits_u, p.gs_u, mode=0, out=out,
                    stream=torch.cuda.current_stream())
    other = make_custom(M, H, I, *spec, seed=M + I + 1)
    odev = swq.to_device(other)
    for rep in range(4):
        out.fill_(float("nan"))
        # another eager call on the same stream (and workspace) between replays
        with torch.cuda.stream(stream):
            swq.forward(*odev, other.bits_g, other.gs_g, other.bits_u, other.gs_u, mode=1, stream=stream)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {rep}"
    check(out.float().cpu().numpy().astype(np.float64), oracle_full(p, 0), 0, "graph replay")


def test_graph_replay_after_workspace_growth():
    """A graph captured while the stream's workspace was small keeps using
    that buffer after a larger eager call replaced it: the old buffer is kept
    (not freed), so replays still write the eager result, and memory allocated
    after the growth is never written by them."""
    small = make_custom(300, 512, 384, 4, 64, 8, 32, seed=91)
    big = make_custom(3000, 2048, 1024, 4, 64, 4, 64, seed=92)
    sdev, bdev = swq.to_device(small), swq.to_device(big)
    say("graph replay after workspace growth")
    stream = torch.cuda.Stream()
    swq.swiglu_q_release_workspace()              # start from no workspace on this stream
    with torch.cuda.stream(stream):
        eager = swq.forward(*sdev, 4, 64, 8, 32, mode=1, stream=stream)
    torch.cuda.synchronize()
    ref = eager.clone()
    out = torch.empty_like(eager)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        swq.forward(*sdev, 4, 64, 8, 32, mode=1, out=out, stream=torch.cuda.current_stream())
    with torch.cuda.stream(stream):                # grows (replaces) the stream's workspace
        yb = swq.forward(*bdev, 4, 64, 4, 64, mode=1, stream=stream)
    torch.cuda.synchronize()
    need = swq.swiglu_q_workspace_bytes(300, 512, 384, 4, 64, 8, 32)
    guard = torch.full((need // 4 + 1024,), 7, dtype=torch.int32, device="cuda")
    for rep in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep}"
    assert bool((guard == 7).all().item())
    ms, ns = sample_pairs(3000, 1024, 400, seed=5)
    check(yb.cpu().numpy().astype(np.float64)[ms, ns], oracle_pairs(big, 1, ms, ns), 1, "grown call")
    del g


def test_leading_dimensions():
    """x of shape [2, 3, H] gives the [2, 3, I] result of the same six rows as [6, H]."""
    p = make_custom(6, 512, 200, 4, 64, 4, 64, seed=93)
    dev = swq.to_device(p)
    say("leading dimensions")
    flat = swq.forward(*dev, 4, 64, mode=1)
    shaped = swq.forward(dev[0].view(2, 3, 512), *dev[1:], 4, 64, mode=1)
    torch.cuda.synchronize()
    assert tuple(shaped.shape) == (2, 3, 200)
    assert torch.equal(shaped.view(6, 200), flat)


def test_call_cap_counts_launched_calls():
    """The bisecting cap turns the predicate off after that many launched
    calls, of either path."""
    p = make_custom(4, 256, 64, 4, 64, seed=6)
    dev = swq.to_device(p)
    say("call cap")
    swq.swiglu_q_reset_counts()
    swq.swiglu_q_set_max_calls(2)
    try:
        assert swq.swiglu_q_under_cap() == 1
        swq.forward(*dev, 4, 64)
        assert swq.swiglu_q_under_cap() == 1
        with forced_path(MFMA, 4):
            swq.forward(*dev, 4, 64)
        torch.cuda.synchronize()
        assert swq.swiglu_q_under_cap() == 0
    finally:
        swq.swiglu_q_set_max_calls(-1)
    assert swq.swiglu_q_under_cap() == 1


# Sums of many same-sign products: activations all positive (as after a SiLU
# or ReLU) or all negative, bf16 and binary16, on every path, in the wide
# mode whose bar is the tightest (a dot-product instruction whose sums are
# not rounded to nearest shows here as a one-sided error) and in MATCH, where
# the M = 1 kernel sums with such an instruction (its error must stay inside
# the tie allowance of the 16-bit rounding of gate and up).
SIGN_SHAPES = [(1, 2048, 300, (4, 64, 4, 64)), (1, 1024, 130, (8, 32, 4, 64)), (3, 2048, 129, (4, 64, 8, 32)),
               (8, 2048, 200, (4, 64, 4, 64)), (20, 1024, 77, (4, 64, 4, 64)), (70, 512, 130, (8, 32, 4, 64))]


@pytest.mark.parametrize("sign", ["positive", "negative"])
@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("M,H,I,spec", SIGN_SHAPES, ids=[f"M{m}-H{h}-I{i}" for m, h, i, _ in SIGN_SHAPES])
def test_same_sign_activations(M, H, I, spec, act, sign):
    p = make_custom(M, H, I, *spec, seed=M + H + I, act=act)
    mag = p.x & np.uint16(0x7FFF)
    p.x = mag | np.uint16(0x8000) if sign == "negative" else mag
    for mode in (1, 0):
        say("same-sign x", sign, act, M, H, I, spec, "mode", mode)
        y = device_forward(p, mode)
        check(y, oracle_full(p, mode), mode, f"same-sign {sign} {act} M{M} H{H} mode {mode}")


# x of a wide dynamic range: every element 2^-j (1 + f) with j uniform in
# 0..17, so one 32-input chunk spans the whole window in which x' is exact
# binary16 (2^-17 of its largest element), products meet the dot products
# and MFMAs at very different exponents, and small terms must not be lost
# beside large ones; mixed and one sign, on every path.
WIDE_SHAPES = [(1, 2048, 256, "gemv"), (3, 2048, 128, "gemv"), (8, 2048, 128, "gemv"), (24, 2048, 96, "gemv"),
               (70, 1024, 256, "mfma"), (300, 2048, 160, "mfma")]


@pytest.mark.parametrize("sign", ["mixed", "positive"])
@pytest.mark.parametrize("M,H,I,path", WIDE_SHAPES, ids=[f"M{m}-H{h}-{p}" for m, h, _, p in WIDE_SHAPES])
def test_wide_range_x(M, H, I, path, sign):
    p = make_custom(M, H, I, 4, 64, 4, 64, seed=M + H)
    rng = np.random.default_rng(M * 7 + 17)
    x = np.ldexp(rng.uniform(1, 2, (M, H)), -rng.integers(0, 18, (M, H)))
    if sign == "mixed":
        x *= rng.choice([-1.0, 1.0], (M, H))
    p.x = to_bf16_bits(x.astype(np.float32))
    path = swq.SWQ_PATH_GEMV if path == "gemv" else swq.SWQ_PATH_MFMA
    for mode in (1, 0):
        say("wide-range x", sign, M, H, I, "path", path, "mode", mode)
        y = device_forward(p, mode, path)
        check(y, oracle_full(p, mode), mode, f"wide x {sign} M{M} mode {mode}")


# The few-row kernel takes x' = x when every row's largest magnitude lies in
# [1, 2^10), else scales by each row's power of two: all-positive rows just
# inside (2^9, 2^10) and well outside (2^14) that range, where a chunk's sum
# of 32 such values would not fit binary16 unscaled.
@pytest.mark.parametrize("top", [2.0 ** 9, 2.0 ** 10, 2.0 ** 14])
@pytest.mark.parametrize("act", ["bf16", "f16"])
def test_few_row_unscaled_range_edges(top, act):
    from synth import f16_bits_to_f32, to_f16_bits
    M, H, I = 8, 2048, 96
    p = make_custom(M, H, I, 4, 64, 4, 64, seed=int(np.log2(top)), act=act)
    rng = np.random.default_rng(int(top))
    x = (rng.uniform(0.5, 1.0, (M, H)) * top * (1 - 2.0 ** -9)).astype(np.float32)
    p.x = to_f16_bits(x) if act == "f16" else to_bf16_bits(x)
    assert swq.swiglu_q_staging_bytes(M, H, I, 4, 64, 4, 64) == 0
    for mode in ((0, 1) if act == "bf16" else (1,)):   # (gate sums of 10^5 overflow a binary16 output)
        say("unscaled range edge", top, act, "mode", mode)
        y = device_forward(p, mode, GEMV)
        check(y, oracle_full(p, mode), mode, f"range edge {top} {act} mode {mode}")
