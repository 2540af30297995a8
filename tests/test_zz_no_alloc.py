"""The allocation-free forward (swiglu_q_forward_noalloc) against the
allocating one, through the C ABI: the same kernels on the same inputs, so
the outputs agree bit for bit; two calls in a row on one GPU, the second with
a smaller input, on each path that stages data, and a HIP graph that records
the call on a stream that has no workspace."""
import numpy as np
import pytest
import torch

import quantized_swiglu_forward_amd as swq
from gpu_helpers import check, oracle_full, say
from synth import make_custom

pytestmark = pytest.mark.gpu

# (first, second) shapes: (M, H, I, spec)
PAIRS = [
    ((600, 2048, 1000, (8, 32, 4, 64)), (130, 1024, 300, (4, 64, 4, 64))),     # matrix-matrix path
    ((9, 2048, 300, (4, 64, 4, 64)), (5, 1024, 200, (4, 64, 8, 32))),          # few rows, prep-fed x'
    ((20, 4096, 130, (4, 64, 4, 64)), (17, 2048, 97, (2, 64, 4, 128))),        # two row tiles
    ((6, 512, 200, (4, 64, 4, 64)), (1, 2048, 300, (4, 64, 4, 64))),           # no staging at all
]


def _run(p, mode, noalloc, stream=None):
    dev = swq.to_device(p)
    dt = torch.float32 if mode == 1 else torch.bfloat16
    out = torch.full((p.M, p.I), float("nan"), dtype=dt, device="cuda")
    fn = swq.swiglu_q_forward_noalloc if noalloc else swq.swiglu_q_forward
    rc = fn(*dev, p.M, p.H, p.I, p.bits_g, p.gs_g, p.bits_u, p.gs_u, mode, out, stream)
    assert rc == swq.SWQ_OK, swq.swiglu_q_strerror(rc)
    torch.cuda.synchronize()
    return out


@pytest.fixture(autouse=True, scope="module")
def _device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    swq.lib()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("pair", PAIRS, ids=["mfma", "few-row", "two-tiles", "unstaged"])
def test_noalloc_matches_forward(pair):
    for i, (M, H, I, spec) in enumerate(pair):
        p = make_custom(M, H, I, *spec, seed=M * 7 + H + I)
        mode = (M + i) % 3
        say("noalloc", M, H, I, spec, "mode", mode)
        ref = _run(p, mode, noalloc=False)
        got = _run(p, mode, noalloc=True)
        assert torch.equal(got.view(torch.int16 if mode != 1 else torch.int32),
                           ref.view(torch.int16 if mode != 1 else torch.int32)), (M, H, I)
        check(got.float().cpu().numpy().astype(np.float64), oracle_full(p, mode), mode, f"noalloc M{M}")


def test_noalloc_in_a_graph_on_a_fresh_stream():
    """Recorded into a HIP graph on a stream that never had a workspace (the
    allocating forward would have to allocate there), replayed with eager
    work between the replays: every replay writes the eager result."""
    p = make_custom(300, 1024, 256, 4, 64, 8, 32, seed=11)
    dev = swq.to_device(p)
    say("noalloc graph")
    ref = _run(p, 1, noalloc=False)
    _run(p, 1, noalloc=True)                       # first call on this GPU: the array's address
    stream = torch.cuda.Stream()
    out = torch.empty((p.M, p.I), dtype=torch.float32, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        rc = swq.swiglu_q_forward_noalloc(*dev, p.M, p.H, p.I, 4, 64, 8, 32, 1, out,
                                          torch.cuda.current_stream())
    assert rc == swq.SWQ_OK
    other = make_custom(200, 512, 128, 4, 64, 4, 64, seed=12)
    for rep in range(3):
        out.fill_(float("nan"))
        _run(other, 0, noalloc=True)               # another call through the same array between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep}"
