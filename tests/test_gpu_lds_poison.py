"""Parity through the LDS-poison debug build (libswiglu_q_ldspoison.so): the
same kernels, each filling its LDS with NaN bits (and 2^30 exponents) before
use, so a kernel that read LDS it had not written would fail here.  One case
per kernel and branch: the M = 1 kernel and its several-row form, the
few-row kernel (x' converted by each wave, built in the block, from the
prep kernel, two row tiles, two column tiles, rows longer than one pass), the prep and MFMA kernels (both tile shapes, the
column split, a partial last super-step, the K split: M = 300, H = 2080
takes four splits of 20, 20, 20 and 5 K-steps, M = 48 four splits in
64-row tiles), the linear and the whole MLP."""
import os

import numpy as np
import pytest
import torch

import oracle
import quantized_swiglu_forward_amd as swq
from gpu_helpers import check, skinny_ct, skinny_x, device_forward, oracle_full, oracle_pairs, say
from synth import make_custom, make_down, make_residual

pytestmark = pytest.mark.gpu

POISON = os.path.join(os.path.dirname(swq.LIB_PATH), "libswiglu_q_ldspoison.so")
GEMV_PATH, MFMA_PATH = swq.SWQ_PATH_GEMV, swq.SWQ_PATH_MFMA


@pytest.fixture(autouse=True, scope="module")
def _poison_library():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert os.path.exists(POISON), f"{POISON} is not built"
    saved = swq.lib()
    swq._lib = swq.load_library(POISON)
    try:
        yield
    finally:
        torch.cuda.synchronize()
        swq._lib = saved


CASES = [
    (1, 2048, 5633, (4, 64, 4, 64), GEMV_PATH), (1, 1024, 300, (8, 32, 4, 64), GEMV_PATH),
    (3, 2048, 301, (8, 32, 4, 64), GEMV_PATH), (6, 256, 768, (4, 64, 4, 64), GEMV_PATH),
    (9, 2048, 300, (4, 64, 4, 64), GEMV_PATH), (20, 1024, 130, (4, 64, 4, 64), GEMV_PATH),
    (12, 8192, 64, (4, 64, 8, 32), GEMV_PATH), (6, 256, 768, (4, 64, 4, 64), MFMA_PATH),
    (300, 2080, 257, (8, 32, 4, 32), MFMA_PATH), (700, 1024, 600, (4, 64, 4, 64), MFMA_PATH),
    (48, 2048, 300, (4, 64, 2, 64), MFMA_PATH),   # K split in 64-row tiles
]


@pytest.mark.parametrize("M,H,I,spec,path", CASES, ids=[f"M{c[0]}-H{c[1]}-I{c[2]}-p{c[4]}" for c in CASES])
def test_forward_under_poison(M, H, I, spec, path):
    mode = (M + H) % 3
    p = make_custom(M, H, I, *spec, seed=M + H + I)
    o = oracle_full(p, mode)
    for source in [None] + (["prep"] if path == GEMV_PATH and M > 1 else []):
        say("poison", M, H, I, spec, "mode", mode, "path", path, "x source", source or "default")
        with skinny_x(source):
            y = device_forward(p, mode, path)
        check(y, o, mode, f"poison M{M} H{H} I{I} x source {source}")


@pytest.mark.parametrize("M,H,I", [(8, 2048, 1000), (5, 1024, 72), (24, 2048, 1000), (32, 1024, 40)])
def test_few_row_two_column_tiles_under_poison(M, H, I):
    """Two column tiles per block of the few-row kernel (their partial sums
    in each wave's region, twice the one-tile size), with one and two row
    tiles (M > 16: regions past 64 KB of LDS per block)."""
    p = make_custom(M, H, I, 4, 64, 4, 64, seed=M + I)
    o = oracle_full(p, 1)
    say("poison two column tiles", M, H, I)
    with skinny_ct(2):
        y = device_forward(p, 1, GEMV_PATH)
    check(y, o, 1, f"poison two column tiles M{M} H{H} I{I}")


@pytest.mark.parametrize("source", [None, "prep"])
def test_few_row_row_groups_under_poison(source):
    """Two row groups of 32 on the matrix-vector path, x converted by each
    group's waves or staged for both groups by the prep kernel."""
    p = make_custom(48, 2048, 300, 4, 64, 4, 64, seed=48)
    o = oracle_full(p, 1)
    say("poison row groups", source or "default")
    with skinny_x(source):
        y = device_forward(p, 1, GEMV_PATH)
    check(y, o, 1, f"poison row groups x source {source}")


def test_split_launch_under_poison():
    """256 x 128 tiles over whole rounds and 128 x 128 tiles for the rest."""
    p = make_custom(512, 256, 38400, 4, 64, 4, 64, seed=41)
    say("poison split launch")
    y = device_forward(p, 1, MFMA_PATH)
    rng = np.random.default_rng(3)
    ns = np.concatenate([np.arange(32768 - 64, 32768 + 64), rng.integers(0, 38400, 300)])
    ms = rng.integers(0, 512, ns.size)
    check(y[ms, ns], oracle_pairs(p, 1, ms, ns), 1, "poison split")


@pytest.mark.parametrize("M", [1, 5, 200])
def test_linear_and_mlp_under_poison(M):
    p = make_custom(M, 512, 640, 4, 64, 4, 64, seed=M)
    dev = swq.to_device(p)
    say("poison linear and mlp", M)
    y = swq.linear(dev[0], dev[1], dev[2], dev[3], 4, 64, swq.SWQ_LINEAR_F32)
    torch.cuda.synchronize()
    from oracle import compare
    r, nu = oracle.qmm_pairs(p.x, p.wg, p.sg, p.bg, p.M, p.H, p.I, 4, 64)
    st = compare.evaluate_linear(y.cpu().numpy(), r, nu, 1)
    assert st["ok"], st
    wd, sd, bd = make_down(512, 640, 4, 64, seed=M + 1)
    res = make_residual(M, 512, seed=M + 2)

    def t16(a):
        return torch.from_numpy(a.view("int16")).cuda().view(torch.bfloat16)

    y = swq.mlp(*dev, torch.from_numpy(wd.view("int32")).cuda(), t16(sd), t16(bd), (4, 64), (4, 64), (4, 64),
                residual=t16(res))
    torch.cuda.synchronize()
    r, nu, _, _ = oracle.mlp_pairs(p, wd, sd, bd, 4, 64, 512, res)
    st = compare.evaluate_mlp(y.float().cpu().numpy(), r, nu, 0)
    assert st["ok"], st
