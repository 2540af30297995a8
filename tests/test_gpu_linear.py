"""GPU parity of the quantized linear ``y = x W^T`` (``swiglu_q_linear``,
through the C ABI) against the oracle's float64 sums, on both kernel paths,
even and odd output sizes, both output types; the projection it computes
equals the fused forward's pre-epilogue gate bit for bit; sampled outputs at
the down-projection shapes of the decode and M=2048 prefill models."""
import contextlib

import numpy as np
import pytest
import torch

import oracle
import quantized_swiglu_forward_amd as swq
from gpu_helpers import forced_path, say
from oracle.compare import evaluate_linear
from synth import make_custom

pytestmark = pytest.mark.gpu

GEMV, MFMA = swq.SWQ_PATH_GEMV, swq.SWQ_PATH_MFMA


@pytest.fixture(autouse=True, scope="module")
def _device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    swq.lib()
    yield
    torch.cuda.synchronize()


def device_linear(p, out_mode, path=None, dev=None):
    if dev is None:
        dev = swq.to_device(p)
    x, w, s, b = dev[:4]
    before = [swq.swiglu_q_call_count(q) for q in (GEMV, MFMA)]
    ctx = forced_path(path, p.M) if path is not None else contextlib.nullcontext()
    with ctx:
        y = swq.linear(x, w, s, b, p.bits_g, p.gs_g, out_mode)
    torch.cuda.synchronize()
    after = [swq.swiglu_q_call_count(q) for q in (GEMV, MFMA)]
    if path is not None and p.M > 0:
        assert after[path] == before[path] + 1, (before, after)
    return y.float().cpu().numpy().astype(np.float64)


def check_linear(y, p, out_mode, what, ms=None, ns=None):
    r, nu = oracle.qmm_pairs(p.x, p.wg, p.sg, p.bg, p.M, p.H, p.I, p.bits_g, p.gs_g, ms, ns)
    yy = y.reshape(-1) if ms is None else y[ms, ns]
    st = evaluate_linear(yy, r, nu, out_mode)
    say(what, f"max_err {st['max_err']:.3g} (tol {st['tol']})")
    assert st["ok"], (what, st)


# (M, K, N, bits, gs, path): N even and odd, N = 1 and 2 (an empty or one-row
# up slot), tiles past M and N, both paths and bit widths, row groups of 32 on
# the matrix-vector path, the MFMA path's K split
CASES = [(300, 256, 200, 4, 64, MFMA), (129, 512, 77, 8, 32, MFMA), (64, 1024, 1, 4, 128, MFMA),
         (257, 256, 2, 4, 64, MFMA), (512, 1024, 1000, 4, 64, MFMA), (33, 384, 129, 8, 64, MFMA),
         (1, 2048, 300, 4, 64, GEMV), (1, 5632, 257, 4, 64, GEMV), (3, 1024, 77, 8, 32, GEMV),
         (16, 2048, 130, 4, 64, GEMV), (1, 256, 1, 4, 32, GEMV), (7, 512, 2, 8, 128, GEMV),
         (129, 512, 77, 2, 64, MFMA), (1, 2048, 133, 2, 32, GEMV), (9, 1024, 65, 2, 128, GEMV),
         (4, 2048, 131, 4, 64, GEMV), (2, 4096, 1, 2, 32, GEMV), (3, 3072, 2, 8, 64, GEMV),
         (40, 2048, 301, 4, 64, GEMV), (100, 1024, 77, 8, 32, GEMV),
         # few MFMA tiles with H >= 2048: K split over blocks (odd N: element stores; 4 | Ig: vector stores)
         (100, 2048, 301, 4, 64, MFMA), (96, 4096, 512, 8, 32, MFMA), (80, 2560, 3, 2, 64, MFMA),
         (70, 8192, 300, 4, 64, MFMA), (70, 2048, 1, 4, 64, MFMA)]


@pytest.mark.parametrize("M,K,N,bits,gs,path", CASES,
                         ids=[f"M{c[0]}-K{c[1]}-N{c[2]}-{c[3]}b{c[4]}-p{c[5]}" for c in CASES])
@pytest.mark.parametrize("out_mode", [swq.SWQ_LINEAR_BF16, swq.SWQ_LINEAR_F32])
def test_linear_against_oracle(M, K, N, bits, gs, path, out_mode):
    p = make_custom(M, K, N, bits, gs, bits, gs, seed=M * 7 + N + out_mode)
    say("linear", M, K, N, bits, gs, "path", path, "out", out_mode)
    y = device_linear(p, out_mode, path)
    check_linear(y, p, out_mode, f"linear M{M} K{K} N{N} path{path} out{out_mode}")


@pytest.mark.parametrize("M,K,N,path", [(200, 512, 301, MFMA), (1, 2048, 133, GEMV), (5, 1024, 64, GEMV),
                                        (1, 8192, 40, GEMV), (3, 2048, 65, GEMV)])
def test_linear_equals_forward_gate_bitwise(M, K, N, path):
    """W's rows in the up slot take the same arithmetic as in the gate slot, so
    the linear's float32 output equals the forward's pre-epilogue gate with W
    as the gate matrix, bit for bit."""
    p = make_custom(M, K, N, 4, 64, 4, 64, seed=N)
    dev = swq.to_device(p)
    say("linear vs gate", M, K, N, path)
    y = device_linear(p, swq.SWQ_LINEAR_F32, path, dev=dev)
    x, w, s, b = dev[:4]
    g, _ = swq.debug_gemm_tensors(x, w, s, b, w, s, b, 4, 64, path=path)
    torch.cuda.synchronize()
    assert np.array_equal(y, g.cpu().numpy().astype(np.float64))


@pytest.mark.parametrize("M,K,N", [(8, 2048, 1201), (13, 1024, 8193)])
def test_linear_few_row_two_column_tiles(M, K, N):
    """The few-row kernel with two column tiles per block, W's rows split
    between the gate and up slots (an odd N leaves the up slot one row
    short): bit for bit the one-tile result with one quad per wave, and
    against the oracle."""
    from gpu_helpers import skinny_ct
    p = make_custom(M, K, N, 4, 64, 4, 64, seed=M + N)
    dev = swq.to_device(p)
    ys = {}
    for ct in (1, 2):
        say("linear column tiles", M, K, N, "ct", ct)
        with skinny_ct(ct, quads=1):
            ys[ct] = device_linear(p, swq.SWQ_LINEAR_F32, GEMV, dev=dev)
    assert np.array_equal(ys[1], ys[2])
    check_linear(ys[2], p, swq.SWQ_LINEAR_F32, f"linear two column tiles M{M} K{K} N{N}")


@pytest.mark.parametrize("M,K,N,path", [(1, 5632, 2048, GEMV), (2048, 14336, 4096, MFMA)],
                         ids=["decode-down-proj", "prefill-down-proj"])
def test_linear_full_size_sampled(M, K, N, path):
    """The down projections of the decode model (hidden 2048, intermediate
    5632) and of the M=2048 prefill model (4096, 14336), 4-bit gs 64: sampled
    outputs against the oracle, corners and tile edges included."""
    p = make_custom(M, K, N, 4, 64, 4, 64, seed=K + N)
    say("linear full size", M, K, N)
    rng = np.random.default_rng(5)
    ms = np.concatenate([[0, M - 1, 0, M - 1], rng.integers(0, M, 400)])
    ns = np.concatenate([[0, 0, N - 1, N - 1], rng.integers(0, N, 400)])
    for out_mode in (swq.SWQ_LINEAR_BF16, swq.SWQ_LINEAR_F32):
        y = device_linear(p, out_mode, path)
        check_linear(y, p, out_mode, f"linear full M{M} out{out_mode}", ms, ns)
