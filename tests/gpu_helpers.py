"""Helpers of the GPU parity tests: run the HIP library through its C ABI on
seeded problems and compare against the CPU oracle."""
from __future__ import annotations

import contextlib
import sys

import numpy as np
import torch

import oracle
import quantized_swiglu_forward_amd as swq
from oracle import compare


def say(*a):
    """Name the case before it touches the device."""
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@contextlib.contextmanager
def forced_path(path, M):
    """Make the dispatcher pick ``path`` for M rows via the threshold setter
    (the default rule afterwards)."""
    if path == swq.SWQ_PATH_GEMV:
        swq.swiglu_q_set_m_threshold(M + 1)
    elif path == swq.SWQ_PATH_MFMA:
        swq.swiglu_q_set_m_threshold(1)
    try:
        yield
    finally:
        swq.swiglu_q_set_m_threshold(-1)


@contextlib.contextmanager
def skinny_x(source):
    """Where the few-row kernel takes x' from: None (the library's choice),
    "prep" or "stage" (SWIGLU_Q_SKINNY_X, read on every call)."""
    import os
    old = os.environ.get("SWIGLU_Q_SKINNY_X")
    if source is None:
        os.environ.pop("SWIGLU_Q_SKINNY_X", None)
    else:
        os.environ["SWIGLU_Q_SKINNY_X"] = source
    try:
        yield
    finally:
        if old is None:
            os.environ.pop("SWIGLU_Q_SKINNY_X", None)
        else:
            os.environ["SWIGLU_Q_SKINNY_X"] = old


@contextlib.contextmanager
def skinny_ct(ct, quads=None):
    """Column tiles per block of the few-row kernel: None (the library's
    choice), 1 or 2 (SWIGLU_Q_SKINNY_CT; 2 applies where the waves convert x
    and a row fits one pass of one chunk quad per wave, and implies one quad
    per wave); ``quads=1`` also gives one tile one quad per wave
    (SWIGLU_Q_SKINNY_QUADS).  Both are read on every call."""
    import os
    want = {"SWIGLU_Q_SKINNY_CT": None if ct is None else str(ct),
            "SWIGLU_Q_SKINNY_QUADS": None if quads is None else str(quads)}
    old = {k: os.environ.get(k) for k in want}
    for k, v in want.items():
        if v is None:
            os.environ.pop(k, None)
        else:
            os.environ[k] = v
    try:
        yield
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def device_forward(prob, mode, path=None, dev=None, expect_path=None):
    """hidden on the GPU as a float64 numpy array [M, I]."""
    if dev is None:
        dev = swq.to_device(prob)
    before = [swq.swiglu_q_call_count(p) for p in (0, 1)]
    ctx = forced_path(path, prob.M) if path is not None else contextlib.nullcontext()
    with ctx:
        out = swq.forward(*dev, prob.bits_g, prob.gs_g, prob.bits_u, prob.gs_u, mode=mode)
    torch.cuda.synchronize()
    after = [swq.swiglu_q_call_count(p) for p in (0, 1)]
    if expect_path is None:
        expect_path = path
    if expect_path is not None and prob.M > 0:
        assert after[expect_path] == before[expect_path] + 1, (before, after)
    return out.float().cpu().numpy().astype(np.float64)


def device_gemm(prob, path=swq.SWQ_PATH_AUTO, dev=None):
    if dev is None:
        dev = swq.to_device(prob)
    g, u = swq.debug_gemm_tensors(*dev, prob.bits_g, prob.gs_g, prob.bits_u, prob.gs_u, path=path)
    torch.cuda.synchronize()
    return g.cpu().numpy().astype(np.float64), u.cpu().numpy().astype(np.float64)


def sample_pairs(M, I, n, seed):
    """Corners, tile edges and random positions of an [M, I] output."""
    rng = np.random.default_rng(seed)
    ms = [0, M - 1, 0, M - 1]
    ns = [0, 0, I - 1, I - 1]
    for e in (31, 32, 63, 64, 127, 128, 255, 256):
        if e < M:
            ms.append(e)
            ns.append(int(rng.integers(0, I)))
        if e < I:
            ms.append(int(rng.integers(0, M)))
            ns.append(e)
    k = max(0, n - len(ms))
    ms = np.concatenate([np.array(ms, np.int64), rng.integers(0, M, k)])
    ns = np.concatenate([np.array(ns, np.int64), rng.integers(0, I, k)])
    return ms, ns


def check(y, o, mode, what):
    st = compare.evaluate(y, o, mode)
    print(f"  {what}: max_err={st['max_err']:.3g} (tol {st['tol']:g}) floor_frac={st['floor_fraction']:.3f} "
          f"max_abs/rms={st['max_abs_over_rms']:.3g} n={st['n']}", flush=True)
    assert st["ok"], (what, st)
    return st


def oracle_full(prob, mode):
    return oracle.swiglu_full(prob, mode)


def oracle_pairs(prob, mode, ms, ns):
    return oracle.swiglu_pairs(prob, mode, ms, ns)
