"""GPU parity of the matrix-matrix path with its K split (few 128 x 128 tiles:
each tile's K-steps shared by several blocks, float32 partial sums added in
order by a second kernel that runs the epilogue) against the oracle, through
the C ABI: every precision mode, ragged M and I (element and vector stores),
mixed and 2/8-bit specs, binary16 activations, the split against the same
call unsplit, and graph replays.  That a case splits is checked from the
workspace size, which includes the partial sums exactly when it does."""
import contextlib
import os

import numpy as np
import pytest
import torch

import quantized_swiglu_forward_amd as swq
from gpu_helpers import check, device_forward, oracle_full, say
from synth import make_custom

pytestmark = pytest.mark.gpu

MFMA = swq.SWQ_PATH_MFMA


@pytest.fixture(autouse=True, scope="module")
def _device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    swq.lib()
    yield
    torch.cuda.synchronize()


@contextlib.contextmanager
def ksplit(cap):
    """At most ``cap`` splits (SWIGLU_Q_MFMA_KSPLIT, read on every call; 0: none)."""
    old = os.environ.get("SWIGLU_Q_MFMA_KSPLIT")
    os.environ["SWIGLU_Q_MFMA_KSPLIT"] = str(cap)
    try:
        yield
    finally:
        if old is None:
            os.environ.pop("SWIGLU_Q_MFMA_KSPLIT", None)
        else:
            os.environ["SWIGLU_Q_MFMA_KSPLIT"] = old


def splits(p):
    with ksplit(0):
        base = swq.swiglu_q_workspace_bytes(p.M, p.H, p.I, p.bits_g, p.gs_g, p.bits_u, p.gs_u)
    return swq.swiglu_q_workspace_bytes(p.M, p.H, p.I, p.bits_g, p.gs_g, p.bits_u, p.gs_u) > base


# (M, H, I, bits_g, gs_g, bits_u, gs_u)
CASES = [
    (70, 2048, 300, 4, 64, 4, 64),      # one row tile, ragged M and I (element stores)
    (128, 2048, 256, 4, 64, 4, 64),     # a full row tile, I % 4 == 0 (vector stores)
    (200, 4096, 520, 8, 32, 4, 128),    # two row tiles, mixed specs, eight splits of 16 steps
    (65, 2048, 1000, 2, 64, 2, 64),     # 2-bit codes
    (129, 2560, 640, 8, 32, 8, 32),     # 8-bit codes, five splits over H = 2560
    (300, 3072, 130, 4, 32, 8, 64),     # three row tiles, I just past one column tile
    (70, 2592, 200, 4, 32, 4, 32),      # 81 K-steps: splits of 20, the last of one step
    (70, 8192, 256, 4, 64, 8, 32),      # 256 K-steps: sixteen splits of 16
    (66, 2048, 1, 4, 64, 4, 64),        # one output column
    # at most 64 rows: 64-row tiles
    (64, 2048, 300, 4, 64, 4, 64),
    (33, 4096, 520, 8, 32, 4, 128),
    (40, 2560, 256, 2, 64, 8, 32),
    (1, 8192, 130, 4, 64, 4, 64),
]


@pytest.mark.parametrize("case", CASES, ids=[f"M{c[0]}_H{c[1]}_I{c[2]}_b{c[3]}g{c[4]}_b{c[5]}g{c[6]}" for c in CASES])
def test_ksplit_against_oracle(case):
    M, H, I, bg, gg, bu, gu = case
    p = make_custom(M, H, I, bg, gg, bu, gu, seed=M * 13 + H + I)
    assert splits(p), case
    dev = swq.to_device(p)
    for mode in (0, 1, 2):
        say("K split", case, "mode", mode)
        y = device_forward(p, mode, MFMA, dev=dev)
        check(y, oracle_full(p, mode), mode, f"K split mode {mode}")
        with ksplit(0):
            say("unsplit", case, "mode", mode)
            y0 = device_forward(p, mode, MFMA, dev=dev)
        # both orders of the same float32 sums round to the oracle's bar; they
        # may differ from each other in the last bits only
        check(y0, oracle_full(p, mode), mode, f"unsplit mode {mode}")
        assert np.max(np.abs(y - y0)) <= 0.01 * max(1.0, float(np.max(np.abs(y0)))), case


def test_ksplit_split_counts_agree():
    """Two, three and the default number of splits all pass the oracle."""
    p = make_custom(96, 4096, 384, 4, 64, 4, 64, seed=5)
    dev = swq.to_device(p)
    o = oracle_full(p, 0)
    for cap in (2, 3, 8):
        with ksplit(cap):
            assert splits(p)
            say("K split cap", cap)
            check(device_forward(p, 0, MFMA, dev=dev), o, 0, f"at most {cap} splits")


def test_ksplit_f16_activations():
    p = make_custom(100, 2048, 130, 4, 64, 4, 64, seed=31, act="f16")
    assert splits(p)
    dev = swq.to_device(p)
    for mode in (0, 1, 2):
        say("K split f16 mode", mode)
        check(device_forward(p, mode, MFMA, dev=dev), oracle_full(p, mode), mode, f"K split f16 mode {mode}")


def test_ksplit_graph_replays():
    """A split call captured in a HIP graph: every replay, with eager calls
    in between, writes the eager result bit for bit (the split sums in a
    fixed order)."""
    p = make_custom(80, 2048, 600, 4, 64, 4, 64, seed=9)
    assert splits(p)
    x, wg, sg, bg, wu, su, bu = swq.to_device(p)
    swq.swiglu_q_set_m_threshold(1)
    try:
        say("K split eager")
        ref = swq.forward(x, wg, sg, bg, wu, su, bu, 4, 64, mode=0)
        torch.cuda.synchronize()
        out = torch.empty_like(ref)
        st = torch.cuda.Stream()
        with torch.cuda.stream(st):
            swq.forward(x, wg, sg, bg, wu, su, bu, 4, 64, mode=0, out=out)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=st):
            swq.forward(x, wg, sg, bg, wu, su, bu, 4, 64, mode=0, out=out)
        for r in range(3):
            out.fill_(0)
            say("K split replay", r)
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), r
            other = swq.forward(x, wg, sg, bg, wu, su, bu, 4, 64, mode=1)
            torch.cuda.synchronize()
            del other
    finally:
        swq.swiglu_q_set_m_threshold(-1)
