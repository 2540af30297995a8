"""GPU parity of the whole MLP ``residual + (silu(x Wg^T) * (x Wu^T)) Wd^T``
(``swiglu_q_mlp``, through the C ABI) against the oracle (its own bf16 hidden
tensor, float64 down projection and residual), on every kernel path of both
halves, odd output sizes, mixed specs, both output types, with and without a
residual; bit for bit equal to the forward followed by the linear; replayed
from a HIP graph; sampled outputs at the M=2048 prefill model's shape."""
import numpy as np
import pytest
import torch

import oracle
import quantized_swiglu_forward_amd as swq
from gpu_helpers import say
from oracle.compare import evaluate_mlp
from synth import make_custom, make_down, make_residual

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    swq.lib()
    yield
    torch.cuda.synchronize()


def _t16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def _t32(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).cuda()


def make_mlp(M, H, I, Ho, spec_g, spec_u, spec_d, residual, seed):
    p = make_custom(M, H, I, *spec_g, *spec_u, seed=seed)
    wd, sd, bd = make_down(Ho, I, *spec_d, seed=seed + 1)
    res = make_residual(M, Ho, seed=seed + 2) if residual else None
    return p, (wd, sd, bd), res


def device_mlp(p, down, res, spec_d, out_mode, dev=None, stream=None):
    if dev is None:
        dev = (*swq.to_device(p), _t32(down[0]), _t16(down[1]), _t16(down[2]),
               _t16(res) if res is not None else None)
    y = swq.mlp(*dev[:10], (p.bits_g, p.gs_g), (p.bits_u, p.gs_u), spec_d, residual=dev[10],
                out_mode=out_mode, stream=stream)
    torch.cuda.synchronize()
    return y, dev


def check(y, p, down, res, spec_d, out_mode, what, ms=None, ns=None):
    Ho = down[0].shape[0]
    r, nu, _, _ = oracle.mlp_pairs(p, *down, *spec_d, Ho, res, ms, ns)
    yy = y.float().cpu().numpy().astype(np.float64)
    yy = yy.reshape(-1) if ms is None else yy[ms, ns]
    st = evaluate_mlp(yy, r, nu, out_mode)
    say(what, f"max_ratio {st['max_ratio']:.3g}, max |dy|/nu {st['max_abs_over_nu']:.3g}")
    assert st["ok"], (what, st)


# (M, H, I, Ho, gate spec, up spec, down spec, residual, out_mode): the forward
# on the M = 1 kernel, its several-row form, the few-row kernel and the MFMA
# kernel; the down projection likewise (its K is I); odd Ho (an uneven split
# of the down matrix between the gate and up slots); every code width
CASES = [
    (1, 2048, 5632, 2048, (4, 64), (4, 64), (4, 64), True, 0),
    (1, 2048, 5632, 2048, (4, 64), (4, 64), (4, 64), False, 1),
    (3, 2048, 1024, 2048, (4, 64), (8, 32), (4, 64), True, 0),
    (6, 256, 768, 256, (4, 64), (4, 64), (4, 64), True, 1),
    (4, 512, 2048, 511, (2, 32), (4, 128), (8, 64), True, 0),
    (300, 512, 384, 512, (8, 32), (4, 64), (8, 32), True, 1),
    (129, 256, 320, 201, (2, 64), (2, 64), (2, 32), False, 0),
    (17, 1024, 2048, 1023, (4, 128), (8, 64), (4, 128), True, 0),
    (64, 2048, 4096, 2048, (4, 64), (4, 64), (4, 64), True, 1),
    # both halves with the MFMA path's K split (few tiles, H and I >= 2048)
    (100, 2048, 2048, 1001, (4, 64), (4, 64), (4, 64), True, 0),
    (80, 2048, 2560, 600, (4, 64), (8, 32), (4, 64), True, 1),
]


@pytest.mark.parametrize("M,H,I,Ho,sg,su,sd,res,out_mode", CASES,
                         ids=[f"M{c[0]}-H{c[1]}-I{c[2]}-Ho{c[3]}-d{c[6][0]}b{c[6][1]}-r{int(c[7])}-o{c[8]}"
                              for c in CASES])
def test_mlp_against_oracle(M, H, I, Ho, sg, su, sd, res, out_mode):
    p, down, r = make_mlp(M, H, I, Ho, sg, su, sd, res, seed=M + H + I + Ho)
    say("mlp", M, H, I, Ho, sg, su, sd, "residual", res, "out", out_mode)
    y, _ = device_mlp(p, down, r, sd, out_mode)
    assert y.shape == (M, Ho)
    check(y, p, down, r, sd, out_mode, f"mlp M{M} H{H} I{I} Ho{Ho}")


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("M,H,I,Ho", [(1, 2048, 2048, 2048), (3, 2048, 1024, 1024), (9, 512, 1024, 515),
                                      (300, 512, 768, 512), (100, 2048, 2048, 1001)])
def test_mlp_equals_forward_then_linear_bitwise(M, H, I, Ho):
    """The whole MLP is the forward in MATCH followed by the linear of the
    down matrix; the residual is added to the linear's float32 sums before
    the one rounding (checked against the host's float32 add and RNE)."""
    spec = (4, 64)
    p, down, r = make_mlp(M, H, I, Ho, spec, spec, spec, True, seed=M * 3 + I)
    say("mlp vs forward + linear", M, H, I, Ho)
    dev = swq.to_device(p)
    wd, sd, bd, res = _t32(down[0]), _t16(down[1]), _t16(down[2]), _t16(r)
    hidden = swq.forward(*dev, *spec, *spec, mode=swq.SWQ_MATCH)
    lin = swq.linear(hidden, wd, sd, bd, *spec, out_mode=swq.SWQ_LINEAR_F32)
    y_plain = swq.mlp(*dev, wd, sd, bd, spec, spec, spec, out_mode=swq.SWQ_LINEAR_F32)
    y_res = swq.mlp(*dev, wd, sd, bd, spec, spec, spec, residual=res, out_mode=swq.SWQ_LINEAR_F32)
    y_res16 = swq.mlp(*dev, wd, sd, bd, spec, spec, spec, residual=res, out_mode=swq.SWQ_LINEAR_BF16)
    torch.cuda.synchronize()
    assert torch.equal(_bits(y_plain), _bits(lin))
    host = lin.cpu() + res.cpu().float()                  # float32 add, as the kernel's epilogue
    assert torch.equal(_bits(y_res.cpu()), _bits(host))
    assert torch.equal(_bits(y_res16.cpu()), _bits(host.to(torch.bfloat16)))


def test_mlp_buffers_grow_and_shrink_between_calls():
    """Calls of growing and shrinking size on one stream (the hidden buffer
    and the workspace grow on demand and are reused) each match the oracle."""
    spec = (4, 64)
    for M, I in ((2, 512), (200, 2048), (5, 1024)):
        p, down, r = make_mlp(M, 512, I, 384, spec, spec, spec, True, seed=M + I)
        say("mlp sizes", M, I)
        y, _ = device_mlp(p, down, r, spec, 0)
        check(y, p, down, r, spec, 0, f"mlp sizes M{M} I{I}")


@pytest.mark.parametrize("M", [1, 40])
def test_mlp_graph_replays_match_eager(M):
    """The whole MLP recorded into a HIP graph after an eager call (so the
    hidden buffer and workspace exist) and replayed several times, with other
    eager calls on the same stream between replays, writes the eager result
    every time."""
    spec = (4, 64)
    p, down, r = make_mlp(M, 1024, 2048, 1024, spec, spec, spec, True, seed=M)
    say("mlp graph", M)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        eager, dev = device_mlp(p, down, r, spec, 0, stream=stream)
    ref = eager.clone()
    out = torch.empty_like(eager)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        swq.mlp(*dev[:10], spec, spec, spec, residual=dev[10], out_mode=0, out=out,
                stream=torch.cuda.current_stream())
    q, qdown, qr = make_mlp(M, 1024, 2048, 1024, spec, spec, spec, True, seed=M + 1)
    for rep in range(4):
        out.fill_(float("nan"))
        with torch.cuda.stream(stream):
            device_mlp(q, qdown, qr, spec, 1, stream=stream)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(ref)), f"replay {rep}"
    check(out, p, down, r, spec, 0, "mlp graph replay")


def test_mlp_full_size_sampled():
    """The M=2048 prefill model's MLP (H=4096, I=14336, 4-bit gs64 gate, up
    and down, with a residual): outputs of 8 rows (first, last, random) at
    48 columns each, corners included, against the oracle."""
    M, H, I, Ho = 2048, 4096, 14336, 4096
    spec = (4, 64)
    p, down, r = make_mlp(M, H, I, Ho, spec, spec, spec, True, seed=33)
    say("mlp full size", M, H, I, Ho)
    y, _ = device_mlp(p, down, r, spec, 0)
    rng = np.random.default_rng(34)
    rows = np.concatenate([[0, M - 1], rng.choice(np.arange(1, M - 1), 6, replace=False)])
    ms = np.repeat(rows, 48)
    ns = np.concatenate([np.concatenate([[0, Ho - 1], rng.integers(0, Ho, 46)]) for _ in rows])
    check(y, p, down, r, spec, 0, "mlp full size sampled", ms, ns)
