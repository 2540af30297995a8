"""Parity of the binary16-activation forward (swiglu_q_forward_f16: x, scales
and biases as float16, float16 output) with the oracle, element by element,
on every kernel path: the M = 1 kernel and its several-row form, the few-row
kernel with x converted by its waves, built in its block and staged by the
prep kernel, and the MFMA kernel; all code widths and precision modes, and
magnitudes at the ends of binary16's range."""
import numpy as np
import pytest
import torch

import quantized_swiglu_forward_amd as swq
from gpu_helpers import check, device_forward, oracle_full, say, skinny_x
from synth import make_custom, to_f16_bits

pytestmark = pytest.mark.gpu

GEMV, MFMA = swq.SWQ_PATH_GEMV, swq.SWQ_PATH_MFMA

# (M, H, I, spec, path, x source): x source only matters to the few-row kernel
CASES = [
    (1, 2048, 300, (4, 64, 4, 64), GEMV, None), (1, 1024, 130, (8, 32, 4, 64), GEMV, None),
    (1, 4096, 257, (2, 64, 2, 64), GEMV, None), (3, 2048, 129, (4, 64, 8, 32), GEMV, None),
    (8, 2048, 200, (4, 64, 4, 64), GEMV, None), (13, 1024, 97, (8, 32, 8, 64), GEMV, None),
    (5, 1056, 77, (2, 32, 2, 32), GEMV, None), (6, 1024, 130, (4, 64, 8, 32), GEMV, "stage"),
    (8, 2048, 96, (4, 128, 4, 64), GEMV, "prep"), (17, 2048, 130, (4, 64, 8, 32), GEMV, None),
    (24, 4096, 64, (4, 128, 4, 64), GEMV, None), (9, 8192, 40, (8, 64, 4, 64), GEMV, None),
    (70, 512, 130, (4, 64, 4, 64), MFMA, None), (300, 2080, 257, (8, 32, 4, 32), MFMA, None),
    (129, 1024, 300, (8, 64, 8, 64), MFMA, None), (256, 768, 384, (2, 64, 4, 128), MFMA, None),
]


@pytest.mark.parametrize("M,H,I,spec,path,src", CASES,
                         ids=[f"M{c[0]}-H{c[1]}-I{c[2]}-p{c[4]}-{c[5] or 'auto'}" for c in CASES])
def test_f16_forward(M, H, I, spec, path, src):
    p = make_custom(M, H, I, *spec, seed=M * 13 + H + I, act="f16")
    dev = swq.to_device(p)
    assert dev[0].dtype == torch.float16
    modes = (0, 1, 2) if M in (1, 8, 70) else ((M + H) % 3,)
    for mode in modes:
        say("f16", M, H, I, spec, "path", path, "x source", src or "default", "mode", mode)
        with skinny_x(src):
            y = device_forward(p, mode, path, dev=dev)
        check(y, oracle_full(p, mode), mode, f"f16 M{M} H{H} I{I} mode {mode}")


def _scaled(M, H, I, spec, seed, x_exp, s_exp, bias=None):
    """A binary16 problem with x times 2^x_exp and scales times 2^s_exp
    (biases -8 s, or uniform in [-bias, bias])."""
    from synth import f16_bits_to_f32
    p = make_custom(M, H, I, *spec, seed=seed, act="f16")
    rng = np.random.default_rng(seed)
    x = f16_bits_to_f32(p.x).astype(np.float64) * 2.0 ** x_exp
    p.x = to_f16_bits(x.astype(np.float32))
    for tag in ("g", "u"):
        s = f16_bits_to_f32(getattr(p, "s" + tag)).astype(np.float64) * 2.0 ** s_exp
        setattr(p, "s" + tag, to_f16_bits(s.astype(np.float32)))
        if bias is None:
            b = -8.0 * f16_bits_to_f32(getattr(p, "s" + tag)).astype(np.float64)
        else:
            b = rng.uniform(-bias, bias, s.shape)
        setattr(p, "b" + tag, to_f16_bits(b.astype(np.float32)))
    return p


# x near binary16's largest value and deep in its subnormals; scales from
# 2^-14 below (subnormal scales) to 2^8 above the generator's; large biases
RANGES = [("x-large", 12, 0, None), ("x-subnormal", -18, 0, None), ("s-small", 0, -14, None),
          ("s-large", -4, 8, None), ("bias-1e3", -2, 0, 1e3)]
RANGE_SHAPES = [(1, 2048, 130, GEMV), (3, 2048, 70, GEMV), (9, 2048, 66, GEMV), (20, 1024, 50, GEMV),
                (70, 512, 130, MFMA)]


@pytest.mark.parametrize("law", RANGES, ids=[r[0] for r in RANGES])
@pytest.mark.parametrize("M,H,I,path", RANGE_SHAPES, ids=[f"M{s[0]}-H{s[1]}-p{s[3]}" for s in RANGE_SHAPES])
def test_f16_range(law, M, H, I, path):
    name, x_exp, s_exp, bias = law
    spec = (4, 64, 8, 32)
    p = _scaled(M, H, I, spec, M + H + I, x_exp, s_exp, bias)
    say("f16 range", name, M, H, I, "path", path)
    y = device_forward(p, 1, path)
    check(y, oracle_full(p, 1), 1, f"f16 range {name} M{M}")


def test_f16_mfma_tile_shapes_agree_bitwise():
    """The binary16 MFMA path in 256 x 128 tiles (forced), in 128 x 128 tiles
    and with the library's choice: every output accumulates the same products
    in the same order whatever the tile shape, so all three agree bit for bit,
    and the oracle accepts them (one row tile past 256 and ragged I)."""
    import os
    p = make_custom(300, 1024, 400, 4, 64, 8, 32, seed=77, act="f16")
    dev = swq.to_device(p)
    outs = {}
    for name, env in (("256", "0"), ("128", "1"), ("auto", None)):
        old = os.environ.get("SWIGLU_Q_MFMA_CFG")
        if env is None:
            os.environ.pop("SWIGLU_Q_MFMA_CFG", None)
        else:
            os.environ["SWIGLU_Q_MFMA_CFG"] = env
        try:
            say("f16 tile shape", name)
            outs[name] = device_forward(p, 1, MFMA, dev=dev)
        finally:
            if old is None:
                os.environ.pop("SWIGLU_Q_MFMA_CFG", None)
            else:
                os.environ["SWIGLU_Q_MFMA_CFG"] = old
    assert np.array_equal(outs["256"].view(np.int64), outs["128"].view(np.int64))
    assert np.array_equal(outs["256"].view(np.int64), outs["auto"].view(np.int64))
    check(outs["256"], oracle_full(p, 1), 1, "f16 256-row tiles")
